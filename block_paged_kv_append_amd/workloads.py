"""Seeded synthetic inputs for block-paged KV attention.

This module draws random numbers and lays them out, nothing more: context
lengths, block tables handed out from a seeded permutation of the physical
block pool, slot mappings for newly appended tokens, and the bf16 / fp32 bit
patterns of q, of the K/V block pools and of new K/V rows.  It computes no part
of the attention itself.  The GPU tests, the benchmark and the CPU oracle all
consume the arrays it returns, so both sides see identical inputs.

Shapes follow the block-paged cache of the "Inference Server" pages (page
"Inference Server", section "What's inside", Paged KV cache row: block-paged
per-layer KV in the vLLM/PagedAttention layout):

* K pool ``[num_blocks, num_kv_heads, head_dim // X, 16, X]`` and
  V pool ``[num_blocks, num_kv_heads, head_dim, 16]``, where ``X`` is the
  number of elements in 16 bytes (8 for bf16, 4 for fp32).
* ``block_tables[b, j]`` is the physical block holding tokens
  ``16*j .. 16*j+15`` of sequence ``b``.
* ``slot_mapping[i] = block * 16 + offset`` names where appended token ``i``
  goes; a negative slot means "skip this token".

Values are float32 ``standard_normal`` draws rounded to bf16 with
round-to-nearest-even.  Every slot no sequence can see (unused blocks, the
tail of a sequence's last block, and slots reserved for tokens still to be
appended) is filled with a quiet NaN so that any read of it shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.uint32(0x7FC00000)


# --------------------------------------------------------------------------
# bit patterns
# --------------------------------------------------------------------------
def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "f32": 4}[dtype]


def pack_x(dtype: str) -> int:
    """Elements per 16-byte chunk of the K pool's innermost axis."""
    return 16 // elem_bytes(dtype)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage bits (bf16 with round-to-nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    u = x.view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2**32, so uint32 arithmetic is exact
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """storage bits -> float32 values (exact for both dtypes)."""
    if dtype == "f32":
        return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32)
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def nan_bits(dtype: str):
    return F32_NAN if dtype == "f32" else BF16_NAN


_CHUNK = 1 << 22


def _normal_bits(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """``standard_normal`` float32 draws (times ``scale``) as storage bits, drawn
    in consecutive chunks into one output array (same stream order as a single
    draw; avoids large temporaries)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.uint32)
    work = np.empty(min(n, _CHUNK), dtype=np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = work[: hi - lo]
        rng.standard_normal(out=x, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = to_bits(x, dtype)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# case containers
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeCase:
    """One batched one-token decode call over a block-paged cache."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    softcap: float  # <= 0: off
    window: int  # <= 0: off
    partition_size: int  # split-K partition (tokens); 0: let the library choose
    num_blocks: int
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, MB]
    q: np.ndarray  # bits [B, Hq, D]
    k_pool: np.ndarray  # bits [NB, Hkv, D/X, 16, X]
    v_pool: np.ndarray  # bits [NB, Hkv, D, 16]

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def gqa_group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


@dataclasses.dataclass
class PrefillCase:
    """One chunked-prefill call: append a chunk of new K/V rows through
    ``slot_mapping``, then attend causally over the cached prefix plus the chunk."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    softcap: float
    window: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [B]   total tokens after the append
    q_lens: np.ndarray  # int32 [B]   chunk length n_b (queries = last n_b tokens)
    cu_q_lens: np.ndarray  # int32 [B+1] prefix sums of q_lens
    block_tables: np.ndarray  # int32 [B, MB]
    q: np.ndarray  # bits [Tq, Hq, D]
    k_pool: np.ndarray  # bits, pool before the append
    v_pool: np.ndarray
    k_new: np.ndarray  # bits [T, Hkv, D]  rows to append (T == Tq here)
    v_new: np.ndarray
    slot_mapping: np.ndarray  # int32 [T]

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def gqa_group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def num_q_tokens(self) -> int:
        return int(self.cu_q_lens[-1])


# --------------------------------------------------------------------------
# pool helpers (layout bookkeeping only)
# --------------------------------------------------------------------------
def pool_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str):
    x = pack_x(dtype)
    return ((num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x),
            (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE))


def _poison_slot(k_pool: np.ndarray, v_pool: np.ndarray, block: int, offset: int, dtype: str) -> None:
    nan = nan_bits(dtype)
    k_pool[block, :, :, offset, :] = nan
    v_pool[block, :, :, offset] = nan


def _poison_unused(k_pool, v_pool, tables, visible_lens, num_blocks, dtype):
    """NaN-fill every pool slot that no sequence reads: whole blocks outside all
    tables and the slots of a table block past the sequence's visible length."""
    nan = nan_bits(dtype)
    used = np.zeros(num_blocks, dtype=bool)
    for b, L in enumerate(visible_lens):
        nblk = (int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE
        used[tables[b, :nblk]] = True
    k_pool[~used] = nan
    v_pool[~used] = nan
    for b, L in enumerate(visible_lens):
        L = int(L)
        if L % BLOCK_SIZE:
            last = int(tables[b, L // BLOCK_SIZE])
            for off in range(L % BLOCK_SIZE, BLOCK_SIZE):
                _poison_slot(k_pool, v_pool, last, off, dtype)
    return used


def _pad_tables(tables: np.ndarray, lens, used: np.ndarray) -> None:
    """Point table entries past each sequence's last block at a poisoned block
    (an unused one if any), so that a stray read returns NaN."""
    spare = np.flatnonzero(~used)
    pad = int(spare[0]) if spare.size else 0
    for b, L in enumerate(lens):
        nblk = (int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE
        tables[b, nblk:] = pad


# --------------------------------------------------------------------------
# generic builders
# --------------------------------------------------------------------------
def make_decode_case(
    seed: int,
    lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    *,
    scale: Optional[float] = None,
    softcap: float = 0.0,
    window: int = 0,
    partition_size: int = 0,
    max_blocks_per_seq: Optional[int] = None,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    q_scale: float = 1.0,
    name: str = "decode",
    rng: Optional[np.random.Generator] = None,
) -> DecodeCase:
    """Draw order: (1) lengths (already given or drawn by the caller from the
    same generator), (2) block permutation, (3) q, (4) K pool, (5) V pool."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.shape[0]
    nblk = [(int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in lens]
    need = int(sum(nblk))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(max(nblk) if nblk else 1, 1)
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * need)), need, 1)
    assert num_blocks >= need
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.zeros((B, max_blocks_per_seq), dtype=np.int32)
    nxt = 0
    for b in range(B):
        tables[b, : nblk[b]] = perm[nxt : nxt + nblk[b]]
        nxt += nblk[b]
    q = _normal_bits(rng, (B, num_q_heads, head_dim), dtype, q_scale)
    kshape, vshape = pool_shapes(num_blocks, num_kv_heads, head_dim, dtype)
    k_pool = _normal_bits(rng, kshape, dtype)
    v_pool = _normal_bits(rng, vshape, dtype)
    used = _poison_unused(k_pool, v_pool, tables, lens, num_blocks, dtype)
    _pad_tables(tables, lens, used)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(name, dtype, num_q_heads, num_kv_heads, head_dim, float(scale),
                      float(softcap), int(window), int(partition_size), int(num_blocks),
                      lens, tables, q, k_pool, v_pool)


def make_prefill_case(
    seed: int,
    cached_lens,
    q_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    *,
    shared_prefix_blocks: int = 0,
    scale: Optional[float] = None,
    softcap: float = 0.0,
    window: int = 0,
    max_blocks_per_seq: Optional[int] = None,
    pool_factor: float = 1.25,
    q_scale: float = 1.0,
    name: str = "prefill",
) -> PrefillCase:
    """A chunk of ``q_lens[b]`` new tokens follows ``cached_lens[b]`` cached
    tokens.  The first ``shared_prefix_blocks`` logical blocks of every table are
    the same physical blocks (a shared, refcounted prefix); all other blocks,
    including those that will receive the chunk, are private.

    Draw order: (1) block permutation, (2) q, (3) K pool, (4) V pool,
    (5) new K rows, (6) new V rows.  Chunk slots start out NaN: only the
    append can make them readable."""
    rng = np.random.default_rng(seed)
    cached = np.asarray(cached_lens, dtype=np.int32)
    qlens = np.asarray(q_lens, dtype=np.int32)
    B = cached.shape[0]
    total = cached + qlens
    S = int(shared_prefix_blocks)
    if S:
        assert all(int(c) >= S * BLOCK_SIZE for c in cached), "shared prefix must be fully cached"
    nblk = [(int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in total]
    need = S + sum(n - S for n in nblk)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(nblk) if nblk else 1
    num_blocks = max(int(math.ceil(pool_factor * need)), need, 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.zeros((B, max_blocks_per_seq), dtype=np.int32)
    shared = perm[:S]
    nxt = S
    for b in range(B):
        tables[b, :S] = shared
        cached_blk = (int(cached[b]) + BLOCK_SIZE - 1) // BLOCK_SIZE
        k = cached_blk - S
        tables[b, S:cached_blk] = perm[nxt : nxt + k]
        nxt += k
    for b in range(B):
        cached_blk = (int(cached[b]) + BLOCK_SIZE - 1) // BLOCK_SIZE
        k = nblk[b] - cached_blk
        tables[b, cached_blk : nblk[b]] = perm[nxt : nxt + k]
        nxt += k
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(qlens)
    Tq = int(cu[-1])
    q = _normal_bits(rng, (Tq, num_q_heads, head_dim), dtype, q_scale)
    kshape, vshape = pool_shapes(num_blocks, num_kv_heads, head_dim, dtype)
    k_pool = _normal_bits(rng, kshape, dtype)
    v_pool = _normal_bits(rng, vshape, dtype)
    k_new = _normal_bits(rng, (Tq, num_kv_heads, head_dim), dtype)
    v_new = _normal_bits(rng, (Tq, num_kv_heads, head_dim), dtype)
    # visible before the append = the cached tokens only
    used = _poison_unused(k_pool, v_pool, tables, cached, num_blocks, dtype)
    # chunk blocks hold no cached token yet but are owned by a table: NaN them
    for b in range(B):
        for t in range(int(cached[b]), int(total[b])):
            _poison_slot(k_pool, v_pool, int(tables[b, t // BLOCK_SIZE]), t % BLOCK_SIZE, dtype)
        used[tables[b, : nblk[b]]] = True
    _pad_tables(tables, total, used)
    slots = np.empty(Tq, dtype=np.int32)
    for b in range(B):
        for j in range(int(qlens[b])):
            t = int(cached[b]) + j
            slots[cu[b] + j] = int(tables[b, t // BLOCK_SIZE]) * BLOCK_SIZE + t % BLOCK_SIZE
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PrefillCase(name, dtype, num_q_heads, num_kv_heads, head_dim, float(scale),
                       float(softcap), int(window), int(num_blocks), total.astype(np.int32),
                       qlens, cu, tables, q, k_pool, v_pool, k_new, v_new, slots)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
def tiny_decode_fp32(seed: int = 1, **kw) -> DecodeCase:
    """4 sequences, lengths {17, 40, 64, 100}; 4 q heads on 1 kv head; D 64;
    fp32; pool of 64 blocks assigned by a seeded permutation; scale 1/8."""
    kw.setdefault("name", "tiny_decode_fp32")
    return make_decode_case(seed, [17, 40, 64, 100], 4, 1, 64, "f32", num_blocks=64,
                            max_blocks_per_seq=7, scale=1.0 / 8.0, **kw)


def gemma_decode(seed: int = 2, **kw) -> DecodeCase:
    """32 sequences, lengths uniform in [512, 4096]; 8 q / 2 kv heads; D 256;
    bf16; tanh logit softcap 50; pool 1.25x the blocks needed."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4096 + 1, size=32).astype(np.int32)
    kw.setdefault("name", "gemma_decode")
    kw.setdefault("softcap", 50.0)
    return make_decode_case(seed, lens, 8, 2, 256, "bf16", scale=1.0 / 16.0,
                            max_blocks_per_seq=4096 // BLOCK_SIZE, rng=rng, **kw)


def sliding_window_decode(seed: int = 3, **kw) -> DecodeCase:
    """32 sequences, lengths uniform in [2048, 8192]; window 512; 8 q / 2 kv
    heads; D 256; bf16; scale 1/16; no softcap."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(2048, 8192 + 1, size=32).astype(np.int32)
    kw.setdefault("name", "sliding_window_decode")
    return make_decode_case(seed, lens, 8, 2, 256, "bf16", scale=1.0 / 16.0, window=512,
                            max_blocks_per_seq=8192 // BLOCK_SIZE, rng=rng, **kw)


def long_context_splitk(seed: int = 4, **kw) -> DecodeCase:
    """8 sequences of 32768 tokens; 32 q / 4 kv heads; D 128; bf16; split-K
    into 512-token partitions."""
    kw.setdefault("name", "long_context_splitk")
    return make_decode_case(seed, [32768] * 8, 32, 4, 128, "bf16", scale=1.0 / math.sqrt(128),
                            partition_size=512, max_blocks_per_seq=32768 // BLOCK_SIZE, **kw)


def chunked_prefill_shared_prefix(seed: int = 5, **kw) -> PrefillCase:
    """8 sequences, 2048 cached tokens each, the first 1024 (64 blocks) shared
    by every table, plus a 512-token chunk appended through slot_mapping and
    attended causally; 8 q / 2 kv heads; D 256; bf16; scale 1/16."""
    kw.setdefault("name", "chunked_prefill_shared_prefix")
    return make_prefill_case(seed, [2048] * 8, [512] * 8, 8, 2, 256, "bf16",
                             shared_prefix_blocks=64, scale=1.0 / 16.0, **kw)


def random_bits(seed: int, shape, dtype: str) -> np.ndarray:
    """N(0, 1) draws of ``shape`` as storage bits."""
    return _normal_bits(np.random.default_rng(seed), shape, dtype)


def new_token_rows(case: DecodeCase, seed: int):
    """K and V rows ``[B, Hkv, D]`` (storage bits, N(0, 1)) of each sequence's
    newest token, for a decode tick that appends them."""
    rng = np.random.default_rng(seed)
    shape = (case.num_seqs, case.num_kv_heads, case.head_dim)
    return _normal_bits(rng, shape, case.dtype), _normal_bits(rng, shape, case.dtype)


NAMED = {
    "tiny_decode_fp32": tiny_decode_fp32,
    "gemma_decode": gemma_decode,
    "sliding_window_decode": sliding_window_decode,
    "long_context_splitk": long_context_splitk,
    "chunked_prefill_shared_prefix": chunked_prefill_shared_prefix,
}
