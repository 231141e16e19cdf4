"""HIP graph capture of the library's launches (the pages' engine replays a
captured decode step, one capture per batch-size bucket; page "Inference
Server", section "The engine").  Every replay, with eager work and synchronisation between
replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32

pytestmark = pytest.mark.gpu


def _replays_match(fn, out, n=4):
    fn()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for k in range(n):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           eager.view(torch.int16) if eager.dtype == torch.bfloat16 else eager), k
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work in between


@pytest.mark.parametrize("split", [0, 64])
def test_decode_graph_replay(split):
    c = wl.make_decode_case(501, [3000, 17, 900, 2048, 5, 700], 8, 2, 256, "bf16", softcap=50.0)
    print("\n[case] decode graph split", split, flush=True)
    q, kp, vp = dev(c.q, "bf16"), dev(c.k_pool, "bf16"), dev(c.v_pool, "bf16")
    bt, cl = i32(c.block_tables), i32(c.context_lens)
    out = torch.empty_like(q)
    ws = torch.zeros(pkv.paged_attn_decode_workspace_size(6, 2, 4, 256, c.max_context_len, split),
                     dtype=torch.uint8, device="cuda")

    def fn():
        args = (out, q, kp, vp, bt, cl, c.max_context_len, c.scale, c.softcap, c.window)
        if split:
            pkv.paged_attn_decode_splitk(*args, partition_size=split, workspace=ws)
        else:
            pkv.paged_attn_decode(*args, workspace=ws)

    _replays_match(fn, out)


def test_append_and_prefill_graph_replay():
    p = wl.make_prefill_case(502, [64, 300], [100, 37], 8, 2, 128, "bf16", shared_prefix_blocks=2)
    print("\n[case] append+prefill graph", flush=True)
    kp0, vp0 = dev(p.k_pool, "bf16"), dev(p.v_pool, "bf16")
    kp, vp = kp0.clone(), vp0.clone()
    kn, vn, sl = dev(p.k_new, "bf16"), dev(p.v_new, "bf16"), i32(p.slot_mapping)
    q = dev(p.q, "bf16")
    out = torch.empty_like(q)
    cu, bt, cl = i32(p.cu_q_lens), i32(p.block_tables), i32(p.context_lens)

    def fn():
        kp.copy_(kp0)
        vp.copy_(vp0)
        pkv.paged_kv_append(kn, vn, sl, kp, vp)
        pkv.paged_attn_prefill(out, q, cu, p.max_q_len, kp, vp, bt, cl, p.max_context_len, p.scale)

    _replays_match(fn, out)


@pytest.mark.parametrize("D,P", [(128, 0), (256, 0), (256, 64)])
def test_decode_tick_graph_bucket(D, P):
    """One bucket of 8 rows captured once (pkv_decode_graph) and replayed for
    three ticks of a decode loop with 8, 5 and 3 active sequences: each tick
    writes new q rows, new K/V rows and lengths one longer into the bound
    buffers; inactive rows have length 0.  Every replay against the oracle's
    tick, the pools carried over from tick to tick."""
    final = [300, 17, 900, 3, 64, 700, 31, 2000]
    Bb, Hq, Hkv, T = 8, 8, 2, 3
    case = wl.make_decode_case(510 + D + P, final, Hq, Hkv, D, "bf16", softcap=20.0)
    assert pkv.decode_bucket(5) == Bb and pkv.decode_bucket(8) == Bb
    q = torch.empty((Bb, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.empty((Bb, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    bt = i32(case.block_tables)
    cl = torch.zeros(Bb, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((Bb, Hq), dtype=torch.float32, device="cuda")
    graph = pkv.DecodeGraph(out, q, kn, vn, kp, vp, bt, cl, max(final), case.scale, case.softcap,
                            partition_size=P, lse=lse)
    kr, vr = case.k_pool, case.v_pool
    for t, active in enumerate([8, 5, 3]):
        print(f"\n[case] decode tick graph D={D} P={P} tick {t} active {active}", flush=True)
        lens = np.array([final[b] - T + 1 + t if b < active else 0 for b in range(Bb)],
                        dtype=np.int32)
        q_t = wl.random_bits(520 + t, (Bb, Hq, D), "bf16")
        kn_t = wl.random_bits(530 + t, (Bb, Hkv, D), "bf16")
        vn_t = wl.random_bits(540 + t, (Bb, Hkv, D), "bf16")
        q.copy_(dev(q_t, "bf16"))
        kn.copy_(dev(kn_t, "bf16"))
        vn.copy_(dev(vn_t, "bf16"))
        cl.copy_(i32(lens))
        out.fill_(float("nan"))
        graph.launch()
        torch.cuda.synchronize()
        ref, ref_lse, kr, vr = oracle.decode_append(q_t, kn_t, vn_t, kr, vr, case.block_tables,
                                                    lens, case.scale, case.softcap, 0, "bf16")
        check_close(as_f64(out), ref, "bf16", f"tick {t}")
        check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, f"tick {t}")
        assert (as_f64(out)[active:] == 0).all()
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work in between
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
    graph.close()


def test_decode_graph_rejects_bad_arguments():
    case = wl.make_decode_case(550, [20, 40], 4, 1, 64, "bf16")
    q = dev(case.q, "bf16")
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    kn = torch.zeros((2, 1, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    with pytest.raises(pkv.PkvError):
        pkv.DecodeGraph(out, q, kn, kn, kp, vp, bt, cl, case.max_context_len, case.scale,
                        partition_size=24)
    lib = pkv.load_library()
    assert lib.pkv_decode_graph_launch(None, None) == -1
    lib.pkv_decode_graph_destroy(None)
