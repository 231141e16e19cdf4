"""Pools larger than 4 GiB, through the C ABI: the prefill then addresses its
blocks with per-block buffer descriptors (smaller pools use one descriptor
per pool and 32-bit offsets), and every kernel forms byte offsets beyond
2^32.  A small case is embedded in pools of 600000 blocks (4.9 GB each at
2 kv heads x head_dim 128, 9.8 GB at head_dim 256, bf16) at block ids near
the end of the pool; the results must equal the oracle's on the small case
(append bit-exact, attention to the bf16 tolerance)."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32

pytestmark = pytest.mark.gpu

BIG_NB = 600_000


def _embed(case, dtype):
    """The case's pools copied into pools of BIG_NB blocks (NaN elsewhere) at
    ids BIG_NB - 1 - 997 i; returns the big pools and the id map."""
    nb = case.k_pool.shape[0]
    ids = np.array([BIG_NB - 1 - 997 * i for i in range(nb)], dtype=np.int64)
    kp_small, vp_small = dev(case.k_pool, dtype), dev(case.v_pool, dtype)
    kp = torch.full((BIG_NB,) + tuple(kp_small.shape[1:]), float("nan"), dtype=kp_small.dtype,
                    device="cuda")
    vp = torch.full((BIG_NB,) + tuple(vp_small.shape[1:]), float("nan"), dtype=vp_small.dtype,
                    device="cuda")
    idx = torch.from_numpy(ids).cuda()
    kp[idx] = kp_small
    vp[idx] = vp_small
    return kp, vp, ids


@pytest.mark.parametrize("cap", [0.0, 50.0])
def test_prefill_head_dim_256_in_pools_over_4gib(cap):
    """head_dim 256 through per-block descriptors (9.8 GB pools), with and
    without softcap: ragged chunks over cached prefixes, a window, against the
    oracle."""
    case = wl.make_prefill_case(73, [100, 520, 0], [40, 77, 130], 8, 2, 256, "bf16", softcap=cap,
                                window=300, q_scale=4.0)
    print("\n[case] pools over 4 GiB: prefill at head_dim 256, softcap", cap, flush=True)
    kp, vp, ids = _embed(case, "bf16")
    assert (BIG_NB * 2 * 256 * 16 * 2) > (1 << 32)
    bt = ids[case.block_tables]
    slots = case.slot_mapping.astype(np.int64)
    big_slots = np.where(slots >= 0, ids[np.maximum(slots, 0) // 16] * 16 + slots % 16, -1)
    pkv.paged_kv_append(dev(case.k_new, "bf16"), dev(case.v_new, "bf16"), i32(big_slots), kp, vp)
    q = dev(case.q, "bf16")
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attn_prefill(out, q, i32(case.cu_q_lens), case.max_q_len, kp, vp, i32(bt),
                           i32(case.context_lens), case.max_context_len, case.scale, case.softcap,
                           case.window, lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool, "bf16")
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(as_f64(out), ref, "bf16", f"prefill D256 cap {cap}, pools over 4 GiB")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"prefill D256 cap {cap}, pools over 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()


def test_prefill_append_and_decode_in_pools_over_4gib():
    case = wl.make_prefill_case(71, [40, 300], [33, 64], 8, 2, 128, "bf16", softcap=30.0)
    assert (BIG_NB * 2 * 128 * 16 * 2) > (1 << 32)
    print("\n[case] pools over 4 GiB: prefill", flush=True)
    kp, vp, ids = _embed(case, "bf16")
    bt = ids[case.block_tables]
    slots = case.slot_mapping.astype(np.int64)
    big_slots = np.where(slots >= 0, ids[np.maximum(slots, 0) // 16] * 16 + slots % 16, -1)
    pkv.paged_kv_append(dev(case.k_new, "bf16"), dev(case.v_new, "bf16"), i32(big_slots), kp, vp)
    q = dev(case.q, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pkv.paged_attn_prefill(out, q, i32(case.cu_q_lens), case.max_q_len, kp, vp, i32(bt),
                           i32(case.context_lens), case.max_context_len, case.scale, case.softcap,
                           case.window, lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool, "bf16")
    idx = torch.from_numpy(ids).cuda()
    assert np.array_equal(pkv.to_bits(kp[idx]), kr) and np.array_equal(pkv.to_bits(vp[idx]), vr)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables,
                                  case.context_lens, case.scale, case.softcap, case.window, "bf16")
    check_close(as_f64(out), ref, "bf16", "prefill, pools over 4 GiB")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, "prefill, pools over 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()

    print("[case] pools over 4 GiB: decode (balanced, split-K) and the fused tick", flush=True)
    d = wl.make_decode_case(72, [17, 300, 1000, 64], 8, 2, 128, "bf16", softcap=50.0, window=200)
    kp, vp, ids = _embed(d, "bf16")
    bt = i32(ids[d.block_tables])
    cl = i32(d.context_lens)
    qd = dev(d.q, "bf16")
    ref, ref_lse = oracle.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.scale,
                                 d.softcap, d.window, "bf16")
    for P in (0, 64):
        out = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda")
        args = (out, qd, kp, vp, bt, cl, d.max_context_len, d.scale, d.softcap, d.window)
        if P:
            pkv.paged_attn_decode_splitk(*args, partition_size=P, lse=lse)
        else:
            pkv.paged_attn_decode(*args, lse=lse)
        torch.cuda.synchronize()
        check_close(as_f64(out), ref, "bf16", f"decode P={P}, pools over 4 GiB")
        check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"decode P={P}, pools over 4 GiB")
    kn, vn = wl.new_token_rows(d, 73)
    tref, _, tk, tv = oracle.decode_append(d.q, kn, vn, d.k_pool, d.v_pool, d.block_tables,
                                           d.context_lens, d.scale, d.softcap, d.window, "bf16")
    out = torch.empty_like(qd)
    pkv.paged_attn_decode_append(out, qd, dev(kn, "bf16"), dev(vn, "bf16"), kp, vp, bt, cl,
                                 d.max_context_len, d.scale, d.softcap, d.window)
    torch.cuda.synchronize()
    idx = torch.from_numpy(ids).cuda()
    assert np.array_equal(pkv.to_bits(kp[idx]), tk) and np.array_equal(pkv.to_bits(vp[idx]), tv)
    check_close(as_f64(out), tref, "bf16", "fused tick, pools over 4 GiB")
