"""paged_attn_decode_no_alloc (the decode on the library's static per-GPU
scratch, for callers that cannot allocate) against the workspace entry points
it stands in for, through the C ABI: the same kernels on the same inputs, so
outputs and lse must be bit-identical; one result is also held to the oracle
(|gpu - ref| <= 2e-2 + 1e-2 |ref| for bf16).  Calls come in a row on the one
scratch, each smaller than the one before, so a call that found the previous
call's partials or counters in the scratch would show."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32, oracle_decode

pytestmark = pytest.mark.gpu


def banner(*what):
    print("\n[case]", *what, flush=True)


def _inputs(case):
    return (dev(case.q, case.dtype), dev(case.k_pool, case.dtype), dev(case.v_pool, case.dtype),
            i32(case.block_tables), i32(case.context_lens))


def _no_alloc(case, P):
    q, kp, vp, bt, cl = _inputs(case)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_no_alloc(out, q, kp, vp, bt, cl, case.max_context_len, case.scale,
                                   case.softcap, case.window, partition_size=P, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _with_workspace(case, P):
    q, kp, vp, bt, cl = _inputs(case)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    args = (out, q, kp, vp, bt, cl, case.max_context_len, case.scale, case.softcap, case.window)
    if P:
        pkv.paged_attn_decode_splitk(*args, partition_size=P, lse=lse)
    else:
        pkv.paged_attn_decode(*args, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
        f"{what}: outputs differ from the workspace entry point"


def test_no_alloc_matches_workspace_entry_points():
    rng = np.random.default_rng(91)
    calls = [
        # (what, case, partition_size): each call smaller than the one before
        ("gemma-style, balanced",
         wl.make_decode_case(92, rng.integers(512, 4097, size=32).tolist(), 8, 2, 256, "bf16",
                             scale=1.0 / 16.0, softcap=50.0), 0),
        ("long rows, split-K P=512",
         wl.make_decode_case(93, [9000, 300, 5000, 17], 8, 2, 128, "bf16"), 512),
        ("small ragged, balanced, window",
         wl.make_decode_case(94, [0, 1, 40, 333, 17], 8, 2, 128, "bf16", window=100), 0),
        ("tiny fp32, split-K P=32",
         wl.make_decode_case(95, [17, 40, 64], 4, 1, 64, "f32"), 32),
    ]
    for k, (what, case, P) in enumerate(calls):
        banner("no_alloc", k, what)
        out, lse = _no_alloc(case, P)
        wout, wlse = _with_workspace(case, P)
        _same(out, wout, what)
        assert torch.equal(lse.view(torch.int32), wlse.view(torch.int32)), f"{what}: lse differs"
        ref, ref_lse = oracle_decode(case)
        check_close(as_f64(out), ref, case.dtype, what)
        check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, what)
    # the first call's sizes again, after the smaller ones
    what, case, P = calls[0]
    banner("no_alloc", "again", what)
    out, _ = _no_alloc(case, P)
    wout, _ = _with_workspace(case, P)
    _same(out, wout, what + " (again)")


def test_no_alloc_rejects_sizes_beyond_the_scratch():
    # split-K with 16-token partitions over 64 sequences x 8 kv heads of up to
    # 8192 tokens: 2^18 partials of 16 x 256 floats, far beyond 32.5 MiB
    B, Hkv, G, D, MB = 64, 8, 16, 256, 512
    q = torch.zeros(B, Hkv * G, D, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(1, Hkv, D // 8, 16, 8, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros(1, Hkv, D, 16, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, MB, dtype=torch.int32, device="cuda")
    cl = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_decode_no_alloc(out, q, kp, vp, bt, cl, MB * 16, 0.0625, 0.0, 0,
                                       partition_size=16)
    assert e.value.code == -3 and "static scratch" in str(e.value)
