"""Shared helpers of the GPU parity tests: run a generated case through the
HIP library and compare with the float64 oracle."""
import numpy as np
import torch

import block_paged_kv_append_amd as pkv
import oracle

# Tolerance for bf16 outputs (fp32 accumulation): |gpu - ref| <= 2e-2 + 1e-2 |ref|,
# plus a relative RMS gate well below it (bf16 output rounding alone gives ~2e-3).
BF16_ATOL, BF16_RTOL, BF16_RMS = 2e-2, 1e-2, 1e-2
# fp32 pools are computed with exact fp32 products and fp32 accumulation
# (hardware exp2 / reciprocal: ~1e-6 relative); the gate leaves two decades.
F32_ATOL, F32_RTOL, F32_RMS = 1e-4, 1e-4, 1e-5
# lse is formed from fp32 logits and fp32 sums in both dtypes.
LSE_ATOL = 2e-3


def dev(bits, dtype):
    return pkv.from_bits(bits, dtype, "cuda")


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def as_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, ref, dtype, what=""):
    """Element-wise tolerance, relative RMS gate, and no NaN."""
    atol, rtol, rms = (BF16_ATOL, BF16_RTOL, BF16_RMS) if dtype == "bf16" else \
        (F32_ATOL, F32_RTOL, F32_RMS)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} elements outside "
                           f"{atol} + {rtol}|ref|; max err {err.max():.3e}")
    ref_rms = np.sqrt(np.mean(ref ** 2))
    if ref_rms > 0:
        ratio = np.sqrt(np.mean(err ** 2)) / ref_rms
        assert ratio <= rms, f"{what}: relative RMS error {ratio:.3e} > {rms}"


def check_lse(got, ref, what=""):
    inf_ref = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf_ref), f"{what}: -inf pattern of lse differs"
    d = np.abs(got[~inf_ref] - ref[~inf_ref])
    assert d.size == 0 or d.max() <= LSE_ATOL, f"{what}: lse max err {d.max():.3e}"


def run_decode(case, mode="balanced", partition_size=None, with_lse=True, workspace=None):
    q = dev(case.q, case.dtype)
    kp = dev(case.k_pool, case.dtype)
    vp = dev(case.v_pool, case.dtype)
    bt = i32(case.block_tables)
    cl = i32(case.context_lens)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda") if with_lse else None
    args = (out, q, kp, vp, bt, cl, case.max_context_len, case.scale, case.softcap, case.window)
    if mode == "balanced":
        pkv.paged_attn_decode(*args, lse=lse, workspace=workspace)
    else:
        P = partition_size or case.partition_size
        pkv.paged_attn_decode_splitk(*args, partition_size=P, lse=lse, workspace=workspace)
    torch.cuda.synchronize()
    return as_f64(out), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


def oracle_decode(case):
    return oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables, case.context_lens,
                         case.scale, case.softcap, case.window, case.dtype)


def run_append(case):
    """GPU append of the case's new rows; returns the pools' bits."""
    kp = dev(case.k_pool, case.dtype)
    vp = dev(case.v_pool, case.dtype)
    pkv.paged_kv_append(dev(case.k_new, case.dtype), dev(case.v_new, case.dtype),
                        i32(case.slot_mapping), kp, vp)
    torch.cuda.synchronize()
    return kp, vp


def run_prefill(case, kp, vp, with_lse=True):
    q = dev(case.q, case.dtype)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda") if with_lse else None
    pkv.paged_attn_prefill(out, q, i32(case.cu_q_lens), case.max_q_len, kp, vp,
                           i32(case.block_tables), i32(case.context_lens), case.max_context_len,
                           case.scale, case.softcap, case.window, lse=lse)
    torch.cuda.synchronize()
    return as_f64(out), (lse.cpu().numpy().astype(np.float64) if with_lse else None)
