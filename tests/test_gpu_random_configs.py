"""Seeded random configurations through every decode form, the chunked
prefill (after its append) and the mixed batch, each compared with the
float64 oracle.

Each case draws a batch size, context lengths (empty sequences, single
tokens and block boundaries included), head_dim, GQA group, an optional
window and softcap, a query scale (flat or peaked softmax) and, for the
split-K form, a partition size; the decode runs balanced, split-K, and as a
fused tick (append of the newest token, then decode).  The prefill cases draw
cached and chunk lengths (empty prefixes, one-token chunks, block edges), a
shared prefix, window, softcap, query scale and the pool dtype.  The
mixed-batch cases draw chunk and decode-row counts.  The draws are fixed by the seeds below, so
a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import (as_f64, check_close, check_lse, dev, i32, oracle_decode, run_append,
                              run_decode, run_prefill)

pytestmark = pytest.mark.gpu

DECODE_SEEDS = list(range(900, 924))
MIXED_SEEDS = list(range(950, 958))
PREFILL_SEEDS = list(range(970, 986))


def _banner(*what):
    print("case:", *what, flush=True)


def _draw_lens(rng, B, max_len):
    lens = rng.integers(1, max_len + 1, size=B)
    kinds = rng.integers(0, 6, size=B)
    lens = np.where(kinds == 0, 0, lens)                                   # empty
    lens = np.where(kinds == 1, 1, lens)                                   # one token
    lens = np.where(kinds == 2, 16 * np.maximum(lens // 16, 1), lens)      # block boundary
    lens = np.where(kinds == 3, 16 * np.maximum(lens // 16, 1) + 1, lens)  # one past it
    return [int(x) for x in np.minimum(lens, max_len)]


def _draw_decode(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 41))
    max_len = int(rng.choice([40, 300, 1500]))
    lens = _draw_lens(rng, B, max_len)
    window = int(rng.choice([0, 0, 17, 64, 200]))
    cap = float(rng.choice([0.0, 0.0, 30.0]))
    q_scale = float(rng.choice([1.0, 8.0]))
    P = int(rng.choice([16, 48, 128, 512]))
    case = wl.make_decode_case(seed, lens, G * Hkv, Hkv, D, "bf16", softcap=cap, window=window,
                               q_scale=q_scale)
    return case, P, dict(D=D, G=G, Hkv=Hkv, B=B, window=window, cap=cap, q_scale=q_scale, P=P)


@pytest.mark.parametrize("seed", DECODE_SEEDS)
def test_random_decode_forms(seed):
    case, P, desc = _draw_decode(seed)
    ref, ref_lse = oracle_decode(case)
    for mode, part in (("balanced", None), ("splitk", P)):
        _banner("random decode", seed, mode, desc)
        out, lse = run_decode(case, mode, part)
        check_close(out, ref, "bf16", f"seed {seed} {mode}")
        check_lse(lse, ref_lse, f"seed {seed} {mode}")


@pytest.mark.parametrize("seed", DECODE_SEEDS[::3])
@pytest.mark.parametrize("P", [0, 32])
def test_random_decode_tick(seed, P):
    """The fused tick: the newest token's rows appended at position L - 1 and
    attended to, in one launch; the pools afterwards bit-exact."""
    case, _, desc = _draw_decode(seed)
    k_new, v_new = wl.new_token_rows(case, seed + 1)
    _banner("random tick", seed, P, desc)
    q = dev(case.q, "bf16")
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_append(out, q, dev(k_new, "bf16"), dev(v_new, "bf16"), kp, vp,
                                 i32(case.block_tables), i32(case.context_lens),
                                 case.max_context_len, case.scale, case.softcap, case.window,
                                 partition_size=P, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse, kr, vr = oracle.decode_append(case.q, k_new, v_new, case.k_pool, case.v_pool,
                                                case.block_tables, case.context_lens, case.scale,
                                                case.softcap, case.window, "bf16")
    assert np.array_equal(pkv.to_bits(kp), kr), f"seed {seed}: K pool differs"
    assert np.array_equal(pkv.to_bits(vp), vr), f"seed {seed}: V pool differs"
    check_close(as_f64(out), ref, "bf16", f"tick seed {seed} P {P}")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"tick seed {seed} P {P}")


@pytest.mark.parametrize("seed", MIXED_SEEDS)
def test_random_mixed_batch(seed):
    """paged_attn_mixed over a random split into chunks and decode rows (one
    launch when both are present)."""
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    n_chunks = int(rng.integers(1, 5))
    n_rows = int(rng.integers(0, 12))
    cached = [int(x) for x in rng.integers(0, 600, size=n_chunks + n_rows)]
    chunk = [int(x) for x in rng.integers(1, 200, size=n_chunks)] + [1] * n_rows
    window = int(rng.choice([0, 0, 100]))
    cap = float(rng.choice([0.0, 30.0]))
    case = wl.make_prefill_case(seed, cached, chunk, G * Hkv, Hkv, D, "bf16", softcap=cap,
                                window=window)
    _banner("random mixed", seed, dict(D=D, G=G, Hkv=Hkv, chunks=n_chunks, rows=n_rows,
                                       window=window, cap=cap))
    kp, vp = run_append(case)
    q = dev(case.q, "bf16")
    out = torch.full_like(q, float("nan"))
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    cu = case.cu_q_lens[:n_chunks + 1]
    pkv.paged_attn_mixed(out, q, i32(cu), int(cu[-1]), int(max(chunk[:n_chunks])), kp, vp,
                         i32(case.block_tables), i32(case.context_lens), case.max_context_len,
                         case.scale, case.softcap, case.window, lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(as_f64(out), ref, "bf16", f"mixed seed {seed}")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"mixed seed {seed}")


@pytest.mark.parametrize("seed", PREFILL_SEEDS)
def test_random_prefill(seed):
    """Append of the chunks' rows (pools bit-exact), then the chunked prefill
    over prefix + chunk, element-wise against the oracle."""
    rng = np.random.default_rng(seed)
    dtype = "f32" if seed % 4 == 3 else "bf16"
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.integers(1, 7))
    shared = int(rng.choice([0, 0, 1, 2]))
    cached = [int(x) for x in rng.integers(0, 700, size=B)]
    kinds = rng.integers(0, 4, size=B)
    cached = [0 if k == 0 else (16 * max(c // 16, 1) if k == 1 else c) for c, k in zip(cached, kinds)]
    cached = [max(c, 16 * shared) for c in cached]
    chunk = [int(x) for x in rng.integers(1, 300, size=B)]
    chunk = [1 if k == 2 else c for c, k in zip(chunk, rng.integers(0, 5, size=B))]
    window = int(rng.choice([0, 0, 33, 200]))
    cap = float(rng.choice([0.0, 30.0]))
    q_scale = float(rng.choice([1.0, 8.0]))
    case = wl.make_prefill_case(seed, cached, chunk, G * Hkv, Hkv, D, dtype,
                                shared_prefix_blocks=shared, softcap=cap, window=window,
                                q_scale=q_scale)
    _banner("random prefill", seed, dict(dtype=dtype, D=D, G=G, Hkv=Hkv, cached=cached,
                                         chunk=chunk, shared=shared, window=window, cap=cap,
                                         q_scale=q_scale))
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           dtype)
    assert np.array_equal(pkv.to_bits(kp), kr), f"seed {seed}: K pool differs"
    assert np.array_equal(pkv.to_bits(vp), vr), f"seed {seed}: V pool differs"
    out, lse = run_prefill(case, kp, vp)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, dtype)
    check_close(out, ref, dtype, f"prefill seed {seed}")
    check_lse(lse, ref_lse, f"prefill seed {seed}")
