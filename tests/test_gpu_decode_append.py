"""GPU parity of the fused decode tick (paged_attn_decode_append) against the
float64 oracle's append-then-decode, on identical seeded inputs.

Before each tick the pools' slots for the newest tokens hold NaN, so a kernel
that read the pool there instead of the new rows would fail the NaN check.
Pools after the tick must match the oracle's bit for bit; outputs to the bf16
(or fp32) tolerance; and the fused launch must give exactly what
paged_kv_append followed by paged_attn_decode gives on the GPU.
"""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32
from tests.test_gpu_parity import SMALL_DECODE

pytestmark = pytest.mark.gpu

BS = 16


def banner(*what):
    print("\n[case]", *what, flush=True)


def pools_before_tick(case):
    """The case's pools with every newest-token slot set to NaN."""
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    for s in oracle.new_token_slots(case.block_tables, case.context_lens).tolist():
        if s >= 0:
            blk, off = divmod(s, BS)
            kp[blk, :, :, off, :] = wl.nan_bits(case.dtype)
            vp[blk, :, :, off] = wl.nan_bits(case.dtype)
    return kp, vp


def run_tick(case, k_new, v_new, kp_bits, vp_bits, partition_size=0, workspace=None):
    q = dev(case.q, case.dtype)
    kp, vp = dev(kp_bits, case.dtype), dev(vp_bits, case.dtype)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_append(out, q, dev(k_new, case.dtype), dev(v_new, case.dtype), kp, vp,
                                 i32(case.block_tables), i32(case.context_lens),
                                 case.max_context_len, case.scale, case.softcap, case.window,
                                 partition_size=partition_size, lse=lse, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse, kp, vp


def check_tick(case, seed, partition_size=0, what=""):
    k_new, v_new = wl.new_token_rows(case, seed)
    kp0, vp0 = pools_before_tick(case)
    out, lse, kp, vp = run_tick(case, k_new, v_new, kp0, vp0, partition_size)
    ref, ref_lse, kr, vr = oracle.decode_append(case.q, k_new, v_new, kp0, vp0,
                                                case.block_tables, case.context_lens, case.scale,
                                                case.softcap, case.window, case.dtype)
    assert np.array_equal(pkv.to_bits(kp), kr), f"{what}: K pool differs"
    assert np.array_equal(pkv.to_bits(vp), vr), f"{what}: V pool differs"
    check_close(as_f64(out), ref, case.dtype, what)
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, what)
    return out, k_new, v_new, kp0, vp0


@pytest.mark.parametrize("spec", SMALL_DECODE,
                         ids=lambda s: f"L{len(s[0])}-G{s[1]//s[2]}-D{s[3]}-{s[4]}-c{s[5]}-w{s[6]}")
@pytest.mark.parametrize("P", [0, 16, 64, 512], ids=["balanced", "splitk16", "splitk64",
                                                     "splitk512"])
def test_decode_append_small(spec, P):
    lens, Hq, Hkv, D, dtype, cap, W = spec
    case = wl.make_decode_case(700 + sum(lens) % 89, lens, Hq, Hkv, D, dtype, softcap=cap, window=W)
    banner("decode_append", P, spec)
    check_tick(case, 701 + D, P, f"decode_append P={P}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_append_block_boundaries_and_empty(D):
    """New tokens that open a block (L % 16 == 1), end one (L % 16 == 0), a
    sequence's first token (L == 1) and empty sequences."""
    lens = [1, 16, 17, 0, 32, 33, 47, 0, 160, 161]
    case = wl.make_decode_case(710 + D, lens, 8, 2, D, "bf16", softcap=30.0)
    for P in (0, 32):
        banner("decode_append boundaries", D, P)
        out, *_ = check_tick(case, 711 + D, P, f"boundaries D={D} P={P}")
        assert (as_f64(out)[3] == 0).all() and (as_f64(out)[7] == 0).all()


def test_decode_append_equals_append_then_decode():
    """The fused launch and the two-call form agree exactly on the GPU."""
    case = wl.make_decode_case(720, [3000, 17, 900, 2048, 5, 700, 1], 8, 2, 256, "bf16",
                               softcap=50.0)
    for P in (0, 64):
        banner("fused vs two calls", P)
        k_new, v_new = wl.new_token_rows(case, 721)
        kp0, vp0 = pools_before_tick(case)
        out, lse, kp, vp = run_tick(case, k_new, v_new, kp0, vp0, P)
        kp2, vp2 = dev(kp0, "bf16"), dev(vp0, "bf16")
        slots = torch.from_numpy(oracle.new_token_slots(case.block_tables, case.context_lens)
                                 .astype(np.int32)).cuda()
        pkv.paged_kv_append(dev(k_new, "bf16"), dev(v_new, "bf16"), slots, kp2, vp2)
        q = dev(case.q, "bf16")
        out2 = torch.empty_like(q)
        lse2 = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        args = (out2, q, kp2, vp2, i32(case.block_tables), i32(case.context_lens),
                case.max_context_len, case.scale, case.softcap, case.window)
        if P:
            pkv.paged_attn_decode_splitk(*args, partition_size=P, lse=lse2)
        else:
            pkv.paged_attn_decode(*args, lse=lse2)
        torch.cuda.synchronize()
        assert torch.equal(kp.view(torch.int16), kp2.view(torch.int16))
        assert torch.equal(vp.view(torch.int16), vp2.view(torch.int16))
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        assert torch.equal(lse, lse2)


def test_decode_append_tiny_fp32():
    case = wl.tiny_decode_fp32()
    for P in (0, 16):
        banner(case.name, "decode_append", P)
        check_tick(case, 731, P, f"tiny fp32 P={P}")


@pytest.mark.parametrize("name,P", [("gemma_decode", 0), ("sliding_window_decode", 0),
                                    ("long_context_splitk", 512)])
def test_decode_append_full(name, P):
    case = wl.NAMED[name]()
    banner(name, "decode_append", P)
    check_tick(case, 740, P, name)


def test_decode_append_rejects_bad_arguments():
    case = wl.make_decode_case(750, [20, 40], 4, 1, 64, "bf16")
    q = dev(case.q, "bf16")
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    kn, vn = (dev(x, "bf16") for x in wl.new_token_rows(case, 751))
    out = torch.empty_like(q)
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    lib = pkv.load_library()
    ws = pkv.decode_workspace(pkv.paged_attn_decode_workspace_size(2, 1, 4, 64, 40, 0), q.device)
    common = (kp.data_ptr(), vp.data_ptr(), case.num_blocks, bt.data_ptr(), bt.shape[1],
              cl.data_ptr(), case.max_context_len, 2, 1, 4, 64, 16, case.scale, 0.0, 0, 0,
              ws.data_ptr(), ws.numel(), pkv.PKV_BF16, None)
    rc = lib.paged_attn_decode_append(out.data_ptr(), None, q.data_ptr(), None, vn.data_ptr(),
                                      *common)
    assert rc == -1 and b"k_new" in lib.pkv_last_error()
    rc = lib.paged_attn_decode_append(out.data_ptr(), None, q.data_ptr(), kn.data_ptr() + 2,
                                      vn.data_ptr(), *common)
    assert rc == -1 and b"aligned" in lib.pkv_last_error()
    with pytest.raises(ValueError):
        pkv.paged_attn_decode_append(out, q, kn[:1], vn[:1], kp, vp, bt, cl,
                                     case.max_context_len, case.scale)
