"""Plain, slow, float64 reference for attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.

What it computes, and where the pages say so
--------------------------------------------
Sources are three web pages about one single-GPU inference engine:

* [engine]  page "Inference Server" (project README mirror), section
  "The engine": a block-paged KV cache with refcounted blocks and
  window-aware sliding layers; paged decode and prefill kernels that read K/V
  through block tables; a split-K decode variant; chunked prefill.
* [inside]  page "Inference Server" (GitHub README), section "What's inside":
  the paged KV cache is block-paged per-layer KV with refcounted blocks and an
  SDPA gather, in the vLLM/PagedAttention layout; the model uses GQA and logit
  softcapping.
* [flow]    page "Inference Server -- Architecture Map", section "How a single
  request flows through the system": long prompts are prefilled one chunk per
  tick; every tick runs one batched decode over all active requests, one new
  token each.

The first read path the pages describe gathers the K/V rows and then runs
standard attention on them [inside]; this
oracle has exactly that structure: gather a sequence's K/V rows through its
block table into contiguous arrays, then apply the textbook definition
softmax(scale * q k^T) v over the visible keys.  Everything is evaluated in
float64 on the exact values stored in bf16 / fp32.

Readings taken where the pages are silent:

* pool layout "vLLM/PagedAttention" [inside]: K pool
  ``[NB, Hkv, D/X, 16, X]`` (X = elements per 16 bytes), V pool
  ``[NB, Hkv, D, 16]``; block size 16;
* ``context_lens[b]`` counts every cached token including the one just
  appended, so the decode query sits at position ``L_b - 1``;
* GQA [inside] maps query head ``h`` to kv head ``h // G`` (contiguous groups);
* softcap [inside] is applied after the scale: ``cap * tanh(scale*q.k / cap)``,
  ``cap <= 0`` meaning off;
* a sliding window of ``W`` [engine] keeps key ``t`` iff ``q_pos - t < W``
  (the last W tokens, the query's own included); ``W <= 0`` means off;
* the AttentionSink policy [inside] keeps the first ``sink`` tokens beside
  the window (StreamingLLM's sink tokens); without a window it changes
  nothing;
* the H2O policy [inside] ranks tokens by the attention they receive: a
  decode step contributes, per token and kv head, the softmax weights of the
  query heads of that group, summed;
* prefill queries are the last ``n_b`` of the ``L_b`` tokens:
  ``q_pos = L_b - n_b + j`` and keys must satisfy ``t <= q_pos``;
* split-K [engine] partitions are anchored at token 0 and merged by
  log-sum-exp; an empty partition carries zero weight;
* a row with no visible key returns 0 with ``lse = -inf``.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 16


# ---------------------------------------------------------------------------
# storage -> values
# ---------------------------------------------------------------------------
def values(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of bf16 (uint16 bits) or fp32 (uint32 bits) storage."""
    if dtype == "bf16":
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _chunk(dtype: str) -> int:
    return {"bf16": 8, "f32": 4}[dtype]


# ---------------------------------------------------------------------------
# [inside] gather through the block table
# ---------------------------------------------------------------------------
def gather_sequence(k_pool, v_pool, table_row, n_tokens: int, kv_head: int, dtype: str):
    """K and V rows ``0 .. n_tokens-1`` of one sequence and kv head, as float64
    ``[n_tokens, D]`` arrays: token ``t`` lives in physical block
    ``table_row[t // 16]`` at offset ``t % 16`` ([engine]: K/V are read through
    block tables; [inside]: PagedAttention layout)."""
    n_blk = (n_tokens + BLOCK - 1) // BLOCK
    ids = np.asarray(table_row[:n_blk], dtype=np.int64)
    D = v_pool.shape[2]
    # K block [D/X, 16, X]: (chunk c, offset o, lane x) holds dim c*X + x of token o
    Kb = values(k_pool[ids, kv_head], dtype)              # [n_blk, D/X, 16, X]
    K = Kb.transpose(0, 2, 1, 3).reshape(n_blk * BLOCK, D)[:n_tokens]
    # V block [D, 16]: (d, o) holds dim d of token o
    Vb = values(v_pool[ids, kv_head], dtype)              # [n_blk, D, 16]
    V = Vb.transpose(0, 2, 1).reshape(n_blk * BLOCK, D)[:n_tokens]
    return K, V


# ---------------------------------------------------------------------------
# masks and scores
# ---------------------------------------------------------------------------
def visible(q_pos: int, n_keys: int, window: int = 0, causal: bool = True,
            sink: int = 0) -> np.ndarray:
    """Boolean mask over keys ``0 .. n_keys-1`` seen by a query at ``q_pos``:
    key ``t`` is kept iff it exists (``t < n_keys``), is not in the future
    (``t <= q_pos``, causal prefill), and, for a window-aware sliding layer
    [engine], lies among the last ``window`` positions (``q_pos - t < window``)
    or, with the AttentionSink policy [inside], among the first ``sink``
    tokens (``t < sink``)."""
    t = np.arange(n_keys)
    keep = np.ones(n_keys, dtype=bool)
    if causal:
        keep &= t <= q_pos
    if window > 0:
        keep &= ((q_pos - t) < window) | (t < sink)
    return keep


def scores(q_rows: np.ndarray, K: np.ndarray, scale: float, softcap: float = 0.0) -> np.ndarray:
    """Logits ``scale * q.k`` and, when ``softcap > 0``, the tanh logit softcap
    [inside] ``softcap * tanh(logit / softcap)``."""
    s = scale * (np.asarray(q_rows, dtype=np.float64) @ K.T)
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    return s


def attend(q_rows, K, V, q_pos, scale, softcap=0.0, window=0, causal=True, sink=0):
    """softmax(scores) @ V over the visible keys, one query row at a time.

    Returns ``out [R, D]`` and the natural-log ``lse [R]``; a row that sees no
    key gets ``out = 0`` and ``lse = -inf``."""
    q_rows = np.atleast_2d(np.asarray(q_rows, dtype=np.float64))
    R, D = q_rows.shape
    n = K.shape[0]
    out = np.zeros((R, D), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    s = scores(q_rows, K, scale, softcap)
    keep = np.stack([visible(int(q_pos[r]), n, window, causal, sink) for r in range(R)])
    any_key = keep.any(axis=1)
    s = np.where(keep, s, -np.inf)
    m = np.where(any_key, s.max(axis=1), 0.0)
    p = np.where(keep, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    ok = any_key
    out[ok] = (p[ok] @ V) / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return out, lse


# ---------------------------------------------------------------------------
# [engine]/[flow] batched one-token decode
# ---------------------------------------------------------------------------
def decode(q, k_pool, v_pool, block_tables, context_lens, scale, softcap=0.0, window=0,
           dtype="bf16", sink=0):
    """One new token per sequence attends over all ``L_b`` cached tokens of its
    sequence (the new token's own K/V included) through the block table.

    ``q`` is storage bits ``[B, Hq, D]``; returns float64 ``out [B, Hq, D]`` and
    ``lse [B, Hq]``."""
    qv = values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = v_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        for g in range(Hkv):
            K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, g, dtype)
            heads = slice(g * G, (g + 1) * G)
            o, ls = attend(qv[b, heads], K, V, [L - 1] * G, scale, softcap, window, causal=True,
                           sink=sink)
            out[b, heads] = o
            lse[b, heads] = ls
    return out, lse


# ---------------------------------------------------------------------------
# [engine] split-K decode: per-partition partials merged by log-sum-exp
# ---------------------------------------------------------------------------
def merge_partials(parts):
    """Merge per-partition results ``(m_p, l_p, o_p)`` of one query row, where
    ``o_p`` is that partition's normalised output, ``l_p`` the sum of
    ``exp(s - m_p)`` over its visible keys and ``m_p`` their max logit.
    Partitions with ``l_p == 0`` see nothing and carry no weight.

    ``out = sum_p w_p o_p / sum_p w_p`` with ``w_p = l_p exp(m_p - M)``,
    ``M = max_p m_p``; ``lse = M + ln sum_p w_p``."""
    live = [(m, l, o) for (m, l, o) in parts if l > 0]
    if not live:
        D = len(parts[0][2]) if parts else 0
        return np.zeros(D), -np.inf
    M = max(m for m, _, _ in live)
    w = np.array([l * math.exp(m - M) for m, l, _ in live])
    O = np.array([o for _, _, o in live])
    return (w @ O) / w.sum(), M + math.log(w.sum())


def decode_splitk(q, k_pool, v_pool, block_tables, context_lens, scale, softcap=0.0, window=0,
                  dtype="bf16", partition_size=512):
    """Decode computed partition by partition: partition ``p`` covers tokens
    ``[p*P, (p+1)*P)`` of the sequence, each yields ``(m_p, l_p, o_p)`` over its
    visible keys, and :func:`merge_partials` combines them.

    Returns ``out [B, Hq, D]``, ``lse [B, Hq]`` and the partials as a dict
    ``{(b, h, p): (m_p, l_p, o_p)}`` for inspection."""
    P = int(partition_size)
    qv = values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = v_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    partials = {}
    for b in range(B):
        L = int(context_lens[b])
        q_pos = L - 1
        for g in range(Hkv):
            K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, g, dtype)
            s_all = scores(qv[b, g * G:(g + 1) * G], K, scale, softcap)
            keep_all = visible(q_pos, L, window, causal=True)
            for hh in range(G):
                h = g * G + hh
                parts = []
                for p in range((L + P - 1) // P):
                    lo, hi = p * P, min((p + 1) * P, L)
                    keep = keep_all[lo:hi]
                    if not keep.any():
                        partials[(b, h, p)] = (-np.inf, 0.0, np.zeros(D))
                        parts.append(partials[(b, h, p)])
                        continue
                    sp = s_all[hh, lo:hi][keep]
                    m = sp.max()
                    e = np.exp(sp - m)
                    l = e.sum()
                    o = (e @ V[lo:hi][keep]) / l
                    partials[(b, h, p)] = (m, l, o)
                    parts.append((m, l, o))
                if parts:
                    out[b, h], lse[b, h] = merge_partials(parts)
    return out, lse, partials


# ---------------------------------------------------------------------------
# [engine]/[flow] chunked prefill
# ---------------------------------------------------------------------------
def prefill(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, scale, softcap=0.0,
            window=0, dtype="bf16"):
    """Sequence ``b`` contributes ``n_b = cu_q_lens[b+1] - cu_q_lens[b]`` query
    rows, the last ``n_b`` of its ``L_b`` tokens; row ``j`` sits at position
    ``L_b - n_b + j`` and attends causally over the cached prefix and the chunk.

    ``q`` is storage bits ``[Tq, Hq, D]``; returns float64 ``out [Tq, Hq, D]``
    and ``lse [Tq, Hq]``."""
    qv = values(q, dtype)
    Tq, Hq, D = qv.shape
    Hkv = v_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    lse = np.full((Tq, Hq), -np.inf, dtype=np.float64)
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        pos = [L - n + j for j in range(n)]
        for g in range(Hkv):
            K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, g, dtype)
            for hh in range(G):
                h = g * G + hh
                o, ls = attend(qv[r0:r1, h], K, V, pos, scale, softcap, window, causal=True)
                out[r0:r1, h] = o
                lse[r0:r1, h] = ls
    return out, lse


# ---------------------------------------------------------------------------
# [engine]/[inside] K/V append into the block pool
# ---------------------------------------------------------------------------
def append(k_new, v_new, slot_mapping, k_pool, v_pool, dtype="bf16"):
    """Copies of the pools with row ``i`` of ``k_new``/``v_new`` (``[T, Hkv, D]``
    storage bits) written to slot ``slot_mapping[i] = block*16 + offset``;
    negative slots are skipped.  A bit copy: no value is converted.

    Raises ``ValueError`` on a duplicate or out-of-range slot."""
    X = _chunk(dtype)
    NB = k_pool.shape[0]
    kp = k_pool.copy()
    vp = v_pool.copy()
    seen = set()
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        if s >= NB * BLOCK:
            raise ValueError(f"slot {s} outside a pool of {NB} blocks")
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        blk, off = divmod(s, BLOCK)
        Hkv, D = k_new.shape[1], k_new.shape[2]
        kp[blk, :, :, off, :] = k_new[i].reshape(Hkv, D // X, X)
        vp[blk, :, :, off] = v_new[i]
    return kp, vp


# ---------------------------------------------------------------------------
# [flow] one decode tick: append every sequence's newest token, then decode
# ---------------------------------------------------------------------------
def new_token_slots(block_tables, context_lens):
    """Slot of each sequence's newest token: position ``L_b - 1`` (``L_b``
    counts it) lives in block ``block_tables[b][(L_b-1) // 16]`` at offset
    ``(L_b-1) % 16`` ([engine]: tokens are found through the block table);
    ``-1`` (nothing to append) when ``L_b == 0``."""
    slots = np.full(len(context_lens), -1, dtype=np.int64)
    for b, L in enumerate(np.asarray(context_lens).tolist()):
        if L > 0:
            slots[b] = int(block_tables[b][(L - 1) // BLOCK]) * BLOCK + (L - 1) % BLOCK
    return slots


def decode_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                  softcap=0.0, window=0, dtype="bf16"):
    """A decode tick as [flow] describes it: each active request's newest
    token (rows ``k_new/v_new [B, Hkv, D]``) is appended to the pool, then one
    batched decode attends over every cached token including it.  Exactly
    :func:`append` at :func:`new_token_slots` followed by :func:`decode`.

    Returns ``out``, ``lse`` and the updated pools' bits."""
    kp, vp = append(k_new, v_new, new_token_slots(block_tables, context_lens), k_pool, v_pool,
                    dtype)
    out, lse = decode(q, kp, vp, block_tables, context_lens, scale, softcap, window, dtype)
    return out, lse, kp, vp


# ---------------------------------------------------------------------------
# [engine] copy-on-write of refcounted shared blocks
# ---------------------------------------------------------------------------
def copy_blocks(src_ids, dst_ids, k_pool, v_pool):
    """Copies of the pools in which block ``dst_ids[i]`` holds what block
    ``src_ids[i]`` held before the call, in both pools, for every kv head and
    all 16 slots ([engine]: blocks are refcounted and shared between
    sequences; one that writes into a shared block first gets its own copy).
    Pairs with ``src == dst`` or an id outside the pool are skipped.

    Raises ``ValueError`` if a destination repeats or is also a source (the
    result would depend on the order of the copies)."""
    NB = k_pool.shape[0]
    src = [int(x) for x in np.asarray(src_ids).tolist()]
    dst = [int(x) for x in np.asarray(dst_ids).tolist()]
    if len(src) != len(dst):
        raise ValueError("src_ids and dst_ids differ in length")
    live = [(s_, d_) for s_, d_ in zip(src, dst) if 0 <= s_ < NB and 0 <= d_ < NB and s_ != d_]
    dsts = [d_ for _, d_ in live]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    if set(dsts) & {s_ for s_, _ in live}:
        raise ValueError("a destination block is also a source")
    kp, vp = k_pool.copy(), v_pool.copy()
    for s_, d_ in live:
        kp[d_] = k_pool[s_]
        vp[d_] = v_pool[s_]
    return kp, vp


# ---------------------------------------------------------------------------
# [inside] eviction statistics: H2O column mass of a decode step
# ---------------------------------------------------------------------------
def column_mass(q, k_pool, v_pool, block_tables, context_lens, scale, softcap=0.0, window=0,
                dtype="bf16", sink=0, length=None):
    """The attention each cached token receives from the decode query of its
    sequence, summed over the query heads that share a kv head: ``mass[b, g,
    t] = sum_{h in group g} p[b, h, t]`` with ``p`` the softmax weights of the
    decode step ([inside]: the H2O eviction policy ranks tokens by the
    attention they accumulate).  Invisible tokens get 0.  Returns float64
    ``[B, Hkv, length]`` (``length`` defaults to the longest context)."""
    qv = values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = v_pool.shape[1]
    G = Hq // Hkv
    n_max = int(max(context_lens)) if len(context_lens) else 0
    length = n_max if length is None else int(length)
    mass = np.zeros((B, Hkv, length), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        keep = visible(L - 1, L, window, True, sink)
        for g in range(Hkv):
            K, _ = gather_sequence(k_pool, v_pool, block_tables[b], L, g, dtype)
            s = scores(qv[b, g * G:(g + 1) * G], K, scale, softcap)   # [G, L]
            s = np.where(keep, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.where(keep, np.exp(s - m), 0.0)
            p /= p.sum(axis=1, keepdims=True)
            mass[b, g, :L] = p.sum(axis=0)
    return mass

