"""GPU parity of the eviction-policy decode variants
(paged_attn_decode_sink_h2o) against the oracle: the AttentionSink mask
(first tokens kept beside the window) and the H2O column mass of the step.

The mass is a sum of softmax weights formed from fp32 logits and the fp32
log-sum-exp; with lse within 2e-3 of the oracle's, each weight is within
about 2e-3 relative, so the gate is |gpu - ref| <= 1e-5 + 5e-3 |ref|, and
every segment's masses must add up to the group size within 1e-3."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32

pytestmark = pytest.mark.gpu

MASS_ATOL, MASS_RTOL = 1e-5, 5e-3


def banner(*what):
    print("\n[case]", *what, flush=True)


def run(case, sink, with_mass=True, stride=None):
    q = dev(case.q, case.dtype)
    kp, vp = dev(case.k_pool, case.dtype), dev(case.v_pool, case.dtype)
    B, Hq, Hkv = case.num_seqs, case.num_q_heads, case.num_kv_heads
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    S = stride or -(-max(case.max_context_len, 1) // 16) * 16
    scores = torch.full((B, Hq, S), float("nan"), device="cuda") if with_mass else None
    mass = torch.full((B, Hkv, S), float("nan"), device="cuda") if with_mass else None
    pkv.paged_attn_decode_sink_h2o(out, q, kp, vp, i32(case.block_tables), i32(case.context_lens),
                                   case.max_context_len, case.scale, case.softcap, case.window,
                                   sink, scores=scores, column_mass=mass, lse=lse)
    torch.cuda.synchronize()
    return (as_f64(out), lse.cpu().numpy().astype(np.float64),
            mass.cpu().numpy().astype(np.float64) if with_mass else None)


def check_mass(got, case, sink, what):
    ref = oracle.column_mass(case.q, case.k_pool, case.v_pool, case.block_tables,
                             case.context_lens, case.scale, case.softcap, case.window,
                             case.dtype, sink, length=got.shape[-1])
    assert not np.isnan(got).any(), f"{what}: NaN in column mass"
    err = np.abs(got - ref)
    bad = err > MASS_ATOL + MASS_RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} mass entries off; max err {err.max():.3e}"
    G = case.gqa_group
    for b, L in enumerate(case.context_lens.tolist()):
        want = G if L > 0 else 0
        assert np.all(np.abs(got[b].sum(axis=-1) - want) <= 1e-3), (what, b)


SPECS = [
    # (lens, Hq, Hkv, D, dtype, softcap, window, sink)
    ([1, 15, 16, 17, 33, 100, 300], 4, 1, 64, "bf16", 0.0, 32, 4),
    ([1, 15, 16, 17, 33, 100, 300], 4, 1, 64, "f32", 0.0, 32, 4),
    ([7, 300, 64, 1000, 129], 8, 2, 128, "bf16", 5.0, 100, 20),
    ([7, 300, 64, 1000, 129], 8, 2, 256, "bf16", 0.0, 17, 40),    # sink blocks > window blocks
    ([2000, 12, 700], 16, 1, 256, "bf16", 30.0, 512, 1),
    ([250, 31, 1, 513], 3, 1, 64, "bf16", 2.0, 64, 64),
    ([40, 17], 2, 1, 128, "f32", 1.5, 16, 9),
    ([4096] * 3 + [17], 8, 2, 256, "bf16", 50.0, 512, 4),
    ([700, 90], 8, 2, 128, "bf16", 0.0, 0, 16),                   # no window: sink is moot
    ([700, 90], 8, 2, 128, "bf16", 0.0, 300, 0),                  # plain window
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"L{len(s[0])}-G{s[1]//s[2]}-D{s[3]}-{s[4]}-w{s[6]}-s{s[7]}")
def test_sink_decode_and_column_mass(spec):
    lens, Hq, Hkv, D, dtype, cap, W, S = spec
    case = wl.make_decode_case(800 + sum(lens) % 83 + S, lens, Hq, Hkv, D, dtype, softcap=cap,
                               window=W)
    banner("sink/h2o", spec)
    out, lse, mass = run(case, S)
    ref, ref_lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                 case.context_lens, case.scale, case.softcap, case.window, dtype,
                                 sink=S)
    check_close(out, ref, dtype, "sink decode")
    check_lse(lse, ref_lse, "sink decode")
    check_mass(mass, case, S, "column mass")


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"L{len(s[0])}-G{s[1]//s[2]}-D{s[3]}-{s[4]}-w{s[6]}-s{s[7]}")
def test_sink_decode_without_mass(spec):
    """AttentionSink alone (no logits, no column mass): the sink tokens stay
    visible beside the window all the same."""
    lens, Hq, Hkv, D, dtype, cap, W, S = spec
    case = wl.make_decode_case(820 + D + S, lens, Hq, Hkv, D, dtype, softcap=cap, window=W)
    banner("sink decode, no mass", spec)
    out, lse, _ = run(case, S, with_mass=False)
    ref, ref_lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                 case.context_lens, case.scale, case.softcap, case.window, dtype,
                                 sink=S)
    check_close(out, ref, dtype, "sink decode, no mass")
    check_lse(lse, ref_lse, "sink decode, no mass")


def test_sliding_window_workload_with_sinks_no_mass_full():
    case = wl.sliding_window_decode()
    banner(case.name, "sink 4, no mass")
    out, lse, _ = run(case, 4, with_mass=False)
    ref, ref_lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                 case.context_lens, case.scale, case.softcap, case.window,
                                 case.dtype, sink=4)
    check_close(out, ref, case.dtype, case.name)
    check_lse(lse, ref_lse, case.name)


def test_sink_decode_without_mass_equals_plain_decode_when_sink_is_zero():
    case = wl.make_decode_case(830, [3000, 17, 900, 2048], 8, 2, 256, "bf16", softcap=50.0,
                               window=512)
    banner("sink 0 vs plain")
    out, lse, _ = run(case, 0, with_mass=False)
    q = dev(case.q, "bf16")
    out2 = torch.empty_like(q)
    lse2 = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode(out2, q, dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16"),
                          i32(case.block_tables), i32(case.context_lens), case.max_context_len,
                          case.scale, case.softcap, case.window, lse=lse2)
    torch.cuda.synchronize()
    assert np.array_equal(out, as_f64(out2)) and np.array_equal(lse, lse2.cpu().numpy())


def test_sliding_window_workload_with_sinks_full():
    case = wl.sliding_window_decode()
    banner(case.name, "sink 4 + column mass")
    out, lse, mass = run(case, 4)
    ref, ref_lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                 case.context_lens, case.scale, case.softcap, case.window,
                                 case.dtype, sink=4)
    check_close(out, ref, case.dtype, case.name)
    check_lse(lse, ref_lse, case.name)
    check_mass(mass, case, 4, case.name)


def test_gemma_workload_column_mass_full():
    case = wl.gemma_decode()
    banner(case.name, "column mass, wider stride")
    out, lse, mass = run(case, 0, stride=4096 + 64)
    check_close(out, oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                   case.context_lens, case.scale, case.softcap, 0,
                                   case.dtype)[0], case.dtype, case.name)
    check_mass(mass, case, 0, case.name)


def test_sink_h2o_rejects_bad_arguments():
    case = wl.make_decode_case(840, [20, 40], 4, 1, 64, "bf16", window=16)
    q = dev(case.q, "bf16")
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty((2, 4), dtype=torch.float32, device="cuda")
    sc = torch.empty((2, 4, 48), device="cuda")
    ms = torch.empty((2, 1, 48), device="cuda")
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    args = (out, q, kp, vp, bt, cl, case.max_context_len, case.scale, 0.0, 16)
    with pytest.raises(pkv.PkvError):
        pkv.paged_attn_decode_sink_h2o(*args, sink_tokens=-1)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode_sink_h2o(*args, column_mass=ms, scores=sc)  # no lse
    with pytest.raises(pkv.PkvError):  # stride below max_context_len
        pkv.paged_attn_decode_sink_h2o(*args, column_mass=ms[..., :32].contiguous(),
                                       scores=sc[..., :32].contiguous(), lse=lse)
