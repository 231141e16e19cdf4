"""GPU parity: the HIP library (through its C ABI) against the float64 oracle on
identical seeded inputs.

* append: bit-exact on the whole pools, NaN poison included;
* attention: every output element within |gpu - ref| <= 2e-2 + 1e-2 |ref|
  for bf16 (1e-4 + 1e-4 |ref| for fp32), a relative-RMS gate, no NaN, and the
  log-sum-exp within 2e-3.

Small cases span several tiles and ragged tails; the named workloads run at
their full sizes in the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import (as_f64, check_close, check_lse, dev, i32, oracle_decode, run_append,
                              run_decode, run_prefill)

pytestmark = pytest.mark.gpu


def banner(*what):
    print("\n[case]", *what, flush=True)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_append_bit_exact(dtype, D):
    case = wl.make_prefill_case(200 + D, [5, 16, 31, 0], [11, 17, 2, 40], 4, 2, D, dtype)
    slots = case.slot_mapping.copy()
    slots[[3, 20]] = -1  # padding tokens
    case.slot_mapping = slots
    banner("append", dtype, D)
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, slots, case.k_pool, case.v_pool, dtype)
    assert np.array_equal(pkv.to_bits(kp).reshape(kr.shape), kr)
    assert np.array_equal(pkv.to_bits(vp).reshape(vr.shape), vr)


def test_append_single_token_per_sequence():
    """The decode-time append: one new token for each of many sequences."""
    case = wl.make_prefill_case(210, list(range(3, 3 + 40 * 7, 7)), [1] * 40, 8, 2, 256, "bf16")
    banner("append decode-style")
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)


def test_append_full_chunked_prefill_workload():
    case = wl.chunked_prefill_shared_prefix()
    banner("append full", case.name)
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           case.dtype)
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)


# ---------------------------------------------------------------------------
# decode (balanced split) and split-K decode on small ragged cases
# ---------------------------------------------------------------------------
SMALL_DECODE = [
    # (lens, Hq, Hkv, D, dtype, softcap, window)
    ([1, 15, 16, 17, 33, 100], 4, 1, 64, "bf16", 0.0, 0),
    ([1, 15, 16, 17, 33, 100], 4, 1, 64, "f32", 0.0, 0),
    ([7, 300, 64, 1000, 129], 8, 2, 128, "bf16", 5.0, 0),
    ([7, 300, 64, 1000, 129], 8, 2, 256, "bf16", 0.0, 100),
    ([250, 31, 1, 513], 16, 16, 128, "bf16", 0.0, 17),
    ([250, 31, 1, 513], 3, 1, 64, "bf16", 2.0, 0),     # group 3: padded head columns
    ([2000, 12, 700], 16, 1, 256, "bf16", 30.0, 0),    # group 16
    ([40, 17], 2, 1, 128, "f32", 1.5, 16),
    ([4096] * 3 + [17], 8, 2, 256, "bf16", 50.0, 512),
    ([5, 70, 300, 1000], 8, 2, 256, "f32", 10.0, 0),   # fp32 at head_dim 256
    ([700, 33, 1], 16, 1, 256, "f32", 0.0, 100),       # fp32, group 16, window
]


@pytest.mark.parametrize("spec", SMALL_DECODE, ids=lambda s: f"L{len(s[0])}-G{s[1]//s[2]}-D{s[3]}-{s[4]}-c{s[5]}-w{s[6]}")
@pytest.mark.parametrize("mode", ["balanced", "splitk16", "splitk64", "splitk512"])
def test_decode_small(spec, mode):
    lens, Hq, Hkv, D, dtype, cap, W = spec
    case = wl.make_decode_case(300 + sum(lens) % 97, lens, Hq, Hkv, D, dtype, softcap=cap, window=W)
    banner("decode", mode, spec)
    if mode == "balanced":
        out, lse = run_decode(case)
    else:
        out, lse = run_decode(case, "splitk", int(mode[6:]))
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, dtype, f"decode {mode}")
    check_lse(lse, ref_lse, f"decode {mode}")


def test_decode_empty_sequences():
    case = wl.make_decode_case(311, [0, 40, 0, 17], 4, 2, 64, "bf16")
    for mode, P in (("balanced", None), ("splitk", 32)):
        banner("decode empty", mode)
        out, lse = run_decode(case, mode, P)
        ref, ref_lse = oracle_decode(case)
        assert (out[0] == 0).all() and (out[2] == 0).all()
        check_close(out, ref, "bf16", mode)
        check_lse(lse, ref_lse, mode)


def test_decode_workspace_reused_across_calls():
    """One workspace, zero-filled once, for many calls in a row (no clearing
    between them: each call leaves its counters at zero), the second with a
    smaller batch, all correct."""
    big = wl.make_decode_case(321, [3000, 17, 900, 2048, 5], 8, 2, 128, "bf16", softcap=20.0)
    small = wl.make_decode_case(322, [100, 1500], 8, 2, 128, "bf16")
    need = max(pkv.paged_attn_decode_workspace_size(5, 2, 4, 128, 3000, 0),
               pkv.paged_attn_decode_workspace_size(5, 2, 4, 128, 3000, 64))
    ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")
    for mode, P in (("balanced", None), ("splitk", 64)):
        for case in (big, small, big):
            banner("decode reuse", mode, case.context_lens.tolist())
            out, lse = run_decode(case, mode, P, workspace=ws)
            ref, ref_lse = oracle_decode(case)
            check_close(out, ref, "bf16", mode)
            check_lse(lse, ref_lse, mode)


def test_decode_without_lse_output():
    case = wl.make_decode_case(331, [77, 1200], 8, 2, 256, "bf16")
    banner("decode no-lse")
    out, _ = run_decode(case, with_lse=False)
    check_close(out, oracle_decode(case)[0], "bf16", "no lse")


def test_decode_poisoned_table_padding_is_never_read():
    """Table entries past each sequence point at NaN blocks; lengths that end
    exactly on a block boundary must not read the next entry."""
    case = wl.make_decode_case(341, [16, 32, 48, 160], 4, 1, 128, "bf16", max_blocks_per_seq=16)
    banner("decode block-boundary")
    out, lse = run_decode(case)
    check_close(out, oracle_decode(case)[0], "bf16", "boundary")


def test_decode_more_workgroups_than_blocks():
    """A max_context_len far above the actual lengths sizes the grid for more
    workgroups than there are blocks (each then gets one block or none); the
    segments split one block per workgroup must still be merged, and leave
    the workspace's counters at zero for the next call."""
    case = wl.make_decode_case(351, [100, 40, 300, 17], 8, 2, 128, "bf16", softcap=10.0,
                               max_blocks_per_seq=256)
    ref, ref_lse = oracle_decode(case)
    q, kp, vp = dev(case.q, "bf16"), dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    ws = torch.zeros(pkv.paged_attn_decode_workspace_size(4, 2, 4, 128, 4096, 0),
                     dtype=torch.uint8, device="cuda")
    for rep in range(3):
        banner("decode N > W", rep)
        out = torch.full_like(q, float("nan"))
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        pkv.paged_attn_decode(out, q, kp, vp, bt, cl, 4096, case.scale, case.softcap, 0,
                              lse=lse, workspace=ws)
        torch.cuda.synchronize()
        check_close(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"N > W {rep}")
        check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"N > W {rep}")
    assert int(ws[:4 * 8].view(torch.int32).abs().sum()) == 0  # counters back at zero


@pytest.mark.gpu
@pytest.mark.parametrize("B", [65, 300])
@pytest.mark.parametrize("mode,P", [("balanced", None), ("splitk", 32)])
def test_decode_large_batch(B, mode, P):
    """Batches past one wave of lengths (65) and past the lengths the decode
    holds in registers (300: sequences 256 and up are read as needed), with
    empty sequences among them, in the balanced and the split-K form."""
    rng = np.random.default_rng(360 + B)
    lens = rng.integers(0, 200, size=B)
    lens[rng.choice(B, size=5, replace=False)] = 0
    case = wl.make_decode_case(361 + B, [int(x) for x in lens], 8, 2, 64, "bf16", softcap=30.0)
    banner("decode large batch", B, mode)
    out, lse = run_decode(case, mode, P)
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, "bf16", f"B={B} {mode}")
    check_lse(lse, ref_lse, f"B={B} {mode}")


@pytest.mark.gpu
def test_decode_at_the_segment_limit():
    """The largest batch one decode call takes: 16384 sequences x 4 kv heads
    = 65536 (sequence, kv head) segments, each with its own merge counter;
    contexts of 0-24 tokens (empty ones and single blocks among them), in the
    balanced and the split-K form on one case."""
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(0, 25, size=16384)]
    case = wl.make_decode_case(31, lens, 8, 4, 64, "bf16", softcap=20.0)
    ref, ref_lse = oracle_decode(case)
    for mode, P in (("balanced", None), ("splitk", 16)):
        banner("decode at the segment limit", mode)
        out, lse = run_decode(case, mode, P)
        check_close(out, ref, "bf16", f"segment limit {mode}")
        check_lse(lse, ref_lse, f"segment limit {mode}")


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------
def test_tiny_decode_fp32():
    case = wl.tiny_decode_fp32()
    for mode, P in (("balanced", None), ("splitk", 16)):
        banner(case.name, mode)
        out, lse = run_decode(case, mode, P)
        ref, ref_lse = oracle_decode(case)
        check_close(out, ref, "f32", mode)
        check_lse(lse, ref_lse, mode)


@pytest.mark.parametrize("q_scale", [1.0, 8.0, 40.0], ids=["plain", "peaked", "softcap-stress"])
def test_gemma_decode_full(q_scale):
    case = wl.gemma_decode(q_scale=q_scale)
    banner(case.name, q_scale)
    out, lse = run_decode(case)
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, "bf16", case.name)
    check_lse(lse, ref_lse, case.name)


@pytest.mark.parametrize("q_scale", [1.0, 8.0], ids=["plain", "peaked"])
def test_sliding_window_decode_full(q_scale):
    case = wl.sliding_window_decode(q_scale=q_scale)
    banner(case.name, q_scale)
    out, lse = run_decode(case)
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, "bf16", case.name)
    check_lse(lse, ref_lse, case.name)


@pytest.mark.parametrize("mode", ["splitk", "balanced"])
def test_long_context_splitk_full(mode):
    case = wl.long_context_splitk(q_scale=8.0)
    banner(case.name, mode)
    out, lse = run_decode(case, mode)
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, "bf16", case.name)
    check_lse(lse, ref_lse, case.name)


def test_long_context_plain_inputs_sampled():
    """Unscaled q: the softmax is nearly flat over 32768 keys; compare every
    output and also the per-partition split-K algebra against the oracle's."""
    case = wl.long_context_splitk()
    banner(case.name, "plain")
    out, lse = run_decode(case, "splitk")
    ref, ref_lse = oracle_decode(case)
    check_close(out, ref, "bf16", case.name)
    check_lse(lse, ref_lse, case.name)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
SMALL_PREFILL = [
    # (cached, chunk, Hq, Hkv, D, dtype, softcap, window, shared_blocks)
    ([0, 16, 33], [40, 16, 5], 4, 1, 64, "bf16", 0.0, 0, 0),
    ([0, 16, 33], [40, 16, 5], 4, 1, 64, "f32", 0.0, 0, 0),
    ([64, 80, 100], [70, 1, 129], 8, 2, 128, "bf16", 10.0, 0, 4),
    ([300, 1], [200, 90], 8, 1, 256, "bf16", 0.0, 64, 0),
    ([48, 48], [77, 3], 2, 2, 128, "bf16", 0.0, 0, 3),      # group 1
    ([20, 5], [33, 64], 16, 1, 64, "bf16", 3.0, 0, 0),      # group 16
    ([20, 5], [33, 64], 16, 8, 128, "bf16", 0.0, 19, 0),    # group 2
    ([513], [250], 8, 2, 256, "f32", 0.0, 0, 0),
]


@pytest.mark.parametrize("spec", SMALL_PREFILL,
                         ids=lambda s: f"G{s[2]//s[3]}-D{s[4]}-{s[5]}-c{s[6]}-w{s[7]}-s{s[8]}")
def test_prefill_small(spec):
    cached, chunk, Hq, Hkv, D, dtype, cap, W, shared = spec
    case = wl.make_prefill_case(400 + D + sum(chunk), cached, chunk, Hq, Hkv, D, dtype,
                                softcap=cap, window=W, shared_prefix_blocks=shared)
    banner("prefill", spec)
    kp, vp = run_append(case)
    out, lse = run_prefill(case, kp, vp)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           dtype)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, dtype)
    check_close(out, ref, dtype, "prefill")
    check_lse(lse, ref_lse, "prefill")


# Stage counts at the edges of the two-wave prefill's interval structure
# (waves w and w + 4 take alternate 32-key stages; copies run one interval
# ahead through a four-stage ring): a single stage (the odd half computes
# nothing), two, three, tails of 1, 15, 16 and 17 keys, and a window whose
# first visible block is not block 0.  Chunks equal to the context make every
# stage a diagonal one.
STAGE_EDGES = [
    # (cached, chunk, Hq, Hkv, D, softcap, window)
    ([0, 0, 0, 0], [5, 16, 31, 32], 8, 2, 256, 0.0, 0),
    ([0, 1, 0, 16], [33, 47, 64, 49], 8, 2, 256, 0.0, 0),
    ([65, 96, 0], [1, 31, 97], 4, 1, 64, 20.0, 0),
    ([200, 31], [40, 70], 8, 2, 128, 0.0, 37),
    ([17, 0], [111, 129], 16, 2, 256, 0.0, 48),
]


@pytest.mark.parametrize("spec", STAGE_EDGES,
                         ids=lambda s: f"D{s[4]}-G{s[2]//s[3]}-{'-'.join(map(str, s[1]))}-w{s[6]}")
def test_prefill_stage_count_edges(spec):
    cached, chunk, Hq, Hkv, D, cap, W = spec
    case = wl.make_prefill_case(900 + D + sum(chunk), cached, chunk, Hq, Hkv, D, "bf16",
                                softcap=cap, window=W)
    banner("prefill stage edges", spec)
    kp, vp = run_append(case)
    out, lse = run_prefill(case, kp, vp)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(out, ref, "bf16", "prefill stage edges")
    check_lse(lse, ref_lse, "prefill stage edges")


@pytest.mark.parametrize("q_scale", [1.0, 8.0], ids=["plain", "peaked"])
def test_chunked_prefill_full(q_scale):
    case = wl.chunked_prefill_shared_prefix(q_scale=q_scale)
    banner(case.name, q_scale)
    kp, vp = run_append(case)
    out, lse = run_prefill(case, kp, vp)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           case.dtype)
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window,
                                  case.dtype)
    check_close(out, ref, "bf16", case.name)
    check_lse(lse, ref_lse, case.name)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
@pytest.mark.parametrize("cap", [0.0, 20.0])
def test_decode_scale_sign(scale, cap):
    """Negative and zero softmax scales (with a window, so masked keys sit
    inside the walked blocks) through every decode form, against the oracle:
    the balanced and split-K decode, the fused tick (balanced and split-K),
    the eviction-policy variant (sink tokens, logits and column mass) and the
    decode rows of a one-launch mixed batch."""
    case = wl.make_decode_case(47, [0, 1, 40, 333, 17], 8, 2, 128, "bf16", scale=scale,
                               softcap=cap, window=100, q_scale=4.0)
    what = f"scale {scale} cap {cap}"
    ref, ref_lse = oracle_decode(case)
    for mode, P in (("balanced", None), ("splitk", 32)):
        banner("decode scale", scale, cap, mode)
        out, lse = run_decode(case, mode, P)
        check_close(out, ref, "bf16", f"{what} {mode}")
        check_lse(lse, ref_lse, f"{what} {mode}")

    # the fused tick: the newest rows appended and attended in one launch
    kn, vn = wl.new_token_rows(case, 48)
    tref, tref_lse, kr, vr = oracle.decode_append(case.q, kn, vn, case.k_pool, case.v_pool,
                                                  case.block_tables, case.context_lens,
                                                  case.scale, case.softcap, case.window, "bf16")
    for P in (0, 32):
        banner("decode scale tick", scale, cap, P)
        q, kp, vp = dev(case.q, "bf16"), dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        pkv.paged_attn_decode_append(out, q, dev(kn, "bf16"), dev(vn, "bf16"), kp, vp,
                                     i32(case.block_tables), i32(case.context_lens),
                                     case.max_context_len, case.scale, case.softcap, case.window,
                                     partition_size=P, lse=lse)
        torch.cuda.synchronize()
        assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
        check_close(as_f64(out), tref, "bf16", f"{what} tick P={P}")
        check_lse(lse.cpu().numpy().astype(np.float64), tref_lse, f"{what} tick P={P}")

    # the eviction-policy variant: 4 sink tokens beside the window, with logits and mass
    banner("decode scale sink/h2o", scale, cap)
    q, kp, vp = dev(case.q, "bf16"), dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    S = -(-case.max_context_len // 16) * 16
    scores = torch.full((case.num_seqs, case.num_q_heads, S), float("nan"), device="cuda")
    mass = torch.full((case.num_seqs, case.num_kv_heads, S), float("nan"), device="cuda")
    pkv.paged_attn_decode_sink_h2o(out, q, kp, vp, i32(case.block_tables), i32(case.context_lens),
                                   case.max_context_len, case.scale, case.softcap, case.window, 4,
                                   scores=scores, column_mass=mass, lse=lse)
    torch.cuda.synchronize()
    sref, sref_lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                   case.context_lens, case.scale, case.softcap, case.window, "bf16",
                                   sink=4)
    check_close(as_f64(out), sref, "bf16", f"{what} sink")
    check_lse(lse.cpu().numpy().astype(np.float64), sref_lse, f"{what} sink")
    mref = oracle.column_mass(case.q, case.k_pool, case.v_pool, case.block_tables,
                              case.context_lens, case.scale, case.softcap, case.window, "bf16", 4,
                              length=S)
    got = mass.cpu().numpy().astype(np.float64)
    assert not np.isnan(got).any() and np.all(np.abs(got - mref) <= 1e-5 + 5e-3 * np.abs(mref))

    # a mixed batch: two chunks, then these sequences as decode rows
    lens = case.context_lens.tolist()
    m = wl.make_prefill_case(49, [60, 200] + [max(L - 1, 0) for L in lens],
                             [70, 33] + [1] * len(lens), 8, 2, 128, "bf16",
                             scale=scale, softcap=cap, window=100, q_scale=4.0)
    banner("decode scale mixed", scale, cap)
    kp, vp = run_append(m)
    q = dev(m.q, "bf16")
    out = torch.full_like(q, float("nan"))
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    cu = m.cu_q_lens[:3]
    pkv.paged_attn_mixed(out, q, i32(cu), int(cu[-1]), 70, kp, vp, i32(m.block_tables),
                         i32(m.context_lens), m.max_context_len, m.scale, m.softcap, m.window,
                         lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(m.k_new, m.v_new, m.slot_mapping, m.k_pool, m.v_pool, "bf16")
    mref, mref_lse = oracle.prefill(m.q, m.cu_q_lens, kr, vr, m.block_tables, m.context_lens,
                                    m.scale, m.softcap, m.window, "bf16")
    check_close(as_f64(out), mref, "bf16", f"{what} mixed")
    check_lse(lse.cpu().numpy().astype(np.float64), mref_lse, f"{what} mixed")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1e-3])
@pytest.mark.parametrize("cap", [0.0, 20.0])
def test_prefill_scale_sign(scale, cap):
    """Negative, zero and tiny softmax scales, with and without softcap (the
    matrix-core prefill folds the scale into its exponent when there is no
    softcap): ragged chunks over cached prefixes, against the oracle."""
    case = wl.make_prefill_case(43, [37, 0, 300], [70, 33, 1], 8, 2, 128, "bf16", scale=scale,
                                softcap=cap, q_scale=4.0)
    banner("prefill scale", scale, cap)
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    out, lse = run_prefill(case, kp, vp)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(out, ref, "bf16", f"scale {scale} cap {cap}")
    check_lse(lse, ref_lse, f"scale {scale} cap {cap}")


@pytest.mark.parametrize("window", [0, 700])
def test_prefill_long_chunk(window):
    """One 3000-token chunk on an empty cache (94 row tiles of one sequence,
    causal across all of them) beside a one-row chunk after 1000 cached
    tokens; append first, then prefill, against the oracle."""
    case = wl.make_prefill_case(41, [0, 1000], [3000, 1], 8, 2, 128, "bf16", window=window)
    banner("prefill long chunk", window)
    kp, vp = run_append(case)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
    out, lse = run_prefill(case, kp, vp)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(out, ref, "bf16", f"long chunk window {window}")
    check_lse(lse, ref_lse, f"long chunk window {window}")


def test_prefill_single_row_equals_decode():
    """A one-token chunk is a decode step: both entry points agree."""
    case = wl.make_prefill_case(451, [100, 700, 31], [1, 1, 1], 8, 2, 256, "bf16", softcap=50.0)
    banner("prefill n=1 vs decode")
    kp, vp = run_append(case)
    out, _ = run_prefill(case, kp, vp)
    q = dev(case.q, "bf16")
    dout = torch.empty_like(q)
    pkv.paged_attn_decode(dout, q, kp, vp, i32(case.block_tables), i32(case.context_lens),
                          case.max_context_len, case.scale, case.softcap, 0)
    torch.cuda.synchronize()
    d = np.abs(out - dout.float().cpu().numpy())
    assert d.max() <= 2e-2

# ---------------------------------------------------------------------------
# mixed batch: decode rows (1-row chunks) and prefill chunks in one launch
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,cap,W", [(128, 0.0, 0), (256, 50.0, 0), (256, 0.0, 300)])
def test_mixed_batch_decode_rows_and_chunks(D, cap, W):
    """One prefill launch over a ragged batch mixing one-row chunks (decode
    rows) with multi-row chunks, against the oracle."""
    cached = [100, 700, 31, 2000, 64, 5, 1500]
    chunk = [1, 300, 1, 1, 64, 1, 1]
    case = wl.make_prefill_case(480 + D + W, cached, chunk, 8, 2, D, "bf16", softcap=cap, window=W)
    banner("mixed batch", D, cap, W)
    kp, vp = run_append(case)
    out, lse = run_prefill(case, kp, vp)
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(out, ref, "bf16", "mixed batch")
    check_lse(lse, ref_lse, "mixed batch")


@pytest.mark.parametrize("D,cap,W", [(128, 0.0, 0), (256, 50.0, 0), (256, 0.0, 300), (64, 0.0, 0)])
def test_mixed_call_chunks_then_decode_rows(D, cap, W):
    """paged_attn_mixed: prefill chunks first, decode rows after them; the
    result equals the oracle's prefill over the whole batch."""
    cached = [700, 64, 33, 100, 2000, 31, 1500, 0]
    chunk = [300, 64, 17, 1, 1, 1, 1, 1]
    P = 3
    case = wl.make_prefill_case(490 + D + W, cached, chunk, 8, 2, D, "bf16", softcap=cap, window=W)
    banner("mixed call", D, cap, W)
    kp, vp = run_append(case)
    q = dev(case.q, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    cu = case.cu_q_lens[:P + 1]
    pkv.paged_attn_mixed(out, q, i32(cu), int(cu[-1]), int(max(chunk[:P])), kp, vp,
                         i32(case.block_tables), i32(case.context_lens), case.max_context_len,
                         case.scale, case.softcap, case.window, lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           "bf16")
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(out.float().cpu().numpy().astype(np.float64), ref, "bf16", "mixed call")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, "mixed call")


def _mixed_call(case, P, dtype, ws=None):
    """paged_attn_mixed over the case's batch: its first P sequences are
    chunks, the rest one-row decode rows (their K/V already appended)."""
    kp, vp = run_append(case)
    q = dev(case.q, dtype)
    out = torch.full_like(q, float("nan"))
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    cu = case.cu_q_lens[:P + 1]
    max_q = int(np.diff(cu).max())
    pkv.paged_attn_mixed(out, q, i32(cu), int(cu[-1]), max_q, kp, vp, i32(case.block_tables),
                         i32(case.context_lens), case.max_context_len, case.scale, case.softcap,
                         case.window, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return as_f64(out), lse.cpu().numpy().astype(np.float64)


def _mixed_ref(case, dtype):
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           dtype)
    return oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables, case.context_lens,
                          case.scale, case.softcap, case.window, dtype)


@pytest.mark.gpu
def test_mixed_call_bench_batch_full():
    """The bench's mixed batch at full size: 4 chunks of 512 new tokens on 2048
    cached ones and 28 decode rows with contexts uniform in [512, 4096], 8 q /
    2 kv heads, D 256, softcap 50, in one launch; twice on one workspace (the
    launch leaves the decode's counters at zero)."""
    rng = np.random.default_rng(6)
    lens = rng.integers(512, 4097, size=28)
    cached = [2048] * 4 + [int(L) - 1 for L in lens]
    chunk = [512] * 4 + [1] * 28
    case = wl.make_prefill_case(6, cached, chunk, 8, 2, 256, "bf16", scale=1.0 / 16.0, softcap=50.0)
    ref, ref_lse = _mixed_ref(case, "bf16")
    ws = torch.zeros(pkv.paged_attn_decode_workspace_size(28, 2, 4, 256, case.max_context_len, 0),
                     dtype=torch.uint8, device="cuda")
    for rep in range(2):
        banner("mixed bench batch", rep)
        out, lse = _mixed_call(case, 4, "bf16", ws)
        check_close(out, ref, "bf16", f"mixed bench batch {rep}")
        check_lse(lse, ref_lse, f"mixed bench batch {rep}")
    assert int(ws[:4 * 56].view(torch.int32).abs().sum()) == 0  # counters back at zero


@pytest.mark.gpu
def test_mixed_call_fp32():
    """fp32 pools take the two-launch form of paged_attn_mixed."""
    cached = [100, 40, 300, 17, 0]
    chunk = [50, 24, 1, 1, 1]
    case = wl.make_prefill_case(497, cached, chunk, 4, 1, 64, "f32", softcap=20.0)
    banner("mixed fp32")
    out, lse = _mixed_call(case, 2, "f32")
    ref, ref_lse = _mixed_ref(case, "f32")
    check_close(out, ref, "f32", "mixed fp32")
    check_lse(lse, ref_lse, "mixed fp32")

