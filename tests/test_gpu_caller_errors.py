"""GPU behaviour on two caller mistakes the kernels turn into defined results
instead of reading or writing where they should not, through the C ABI.

* A prefill chunk longer than its context (n_b > L_b): rows at negative
  positions see no key and get out = 0 and lse = -inf, whether the whole
  workgroup's rows sit before the cache or only some of them.
* A decode tick whose context length exceeds max_context_len: the length is
  clamped for the attention, and the fused append writes nothing for that
  sequence (its clamped last position holds an older token)."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32, run_append

pytestmark = pytest.mark.gpu


def banner(*what):
    print("\n[case]", *what, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_rows_before_the_cache(dtype, D):
    # chunk 0: 40 rows over a context of 10 (30 rows at negative positions);
    # chunk 2: 64 rows over 20 (a whole workgroup's rows before the cache)
    case = wl.make_prefill_case(61, [0, 100, 0], [40, 33, 64], 8, 2, D, dtype)
    kp, vp = run_append(case)
    cl = case.context_lens.copy()
    cl[0], cl[2] = 10, 20
    banner("prefill rows before the cache", dtype, D, cl.tolist())
    q = dev(case.q, dtype)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attn_prefill(out, q, i32(case.cu_q_lens), case.max_q_len, kp, vp,
                           i32(case.block_tables), i32(cl), case.max_context_len, case.scale,
                           case.softcap, case.window, lse=lse)
    torch.cuda.synchronize()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           dtype)
    ref, ref_lse = oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables, cl,
                                  case.scale, case.softcap, case.window, dtype)
    got = as_f64(out)
    check_close(got, ref, dtype, "prefill rows before the cache")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, "prefill rows before the cache")
    # the rows before the cache are exactly zero, lse -inf
    neg = np.concatenate([np.arange(0, 30), case.cu_q_lens[2] + np.arange(0, 44)])
    assert np.all(got[neg] == 0.0)
    assert np.all(np.isneginf(lse.cpu().numpy()[neg]))


@pytest.mark.parametrize("P", [0, 32])
def test_decode_tick_length_beyond_max_context_len(P):
    lens = [40, 100, 17]
    case = wl.make_decode_case(62, lens, 8, 2, 128, "bf16", max_blocks_per_seq=10)
    assert case.max_context_len == 100
    kn, vn = wl.new_token_rows(case, 63)
    cl = np.array([40, 130, 17], dtype=np.int32)  # sequence 1 beyond max_context_len
    banner("decode tick beyond max_context_len", P)
    q, kp, vp = dev(case.q, "bf16"), dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    out = torch.empty_like(q)
    pkv.paged_attn_decode_append(out, q, dev(kn, "bf16"), dev(vn, "bf16"), kp, vp,
                                 i32(case.block_tables), i32(cl), 100, case.scale, case.softcap,
                                 case.window, partition_size=P)
    torch.cuda.synchronize()
    # sequences 0 and 2: the ordinary tick; sequence 1: no append, attention
    # over its first 100 tokens
    slots = oracle.new_token_slots(case.block_tables, case.context_lens)
    slots[1] = -1
    kr, vr = oracle.append(kn, vn, slots, case.k_pool, case.v_pool, "bf16")
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
    ref, _ = oracle.decode(case.q, kr, vr, case.block_tables, case.context_lens, case.scale,
                           case.softcap, case.window, "bf16")
    check_close(as_f64(out), ref, "bf16", "tick beyond max_context_len")
