"""HIP graph capture of the library's launches (the pages' engine replays a
captured decode step; page "Inference Server", section "The engine": bucketed
CUDA-graph decode).  Every replay, with eager work and synchronisation between
replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import dev, i32

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
