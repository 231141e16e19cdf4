"""GPU parity of the copy-on-write block copy (paged_kv_copy_blocks) against
the oracle, and a decode tick of two sequences that share a prefix, with the
host allocator preparing the copy-on-write before both append."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
import oracle
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import as_f64, check_close, check_lse, dev, i32

pytestmark = pytest.mark.gpu


def banner(*what):
    print("\n[case]", *what, flush=True)


def random_pools(seed, NB, Hkv, D, dtype):
    kshape, vshape = wl.pool_shapes(NB, Hkv, D, dtype)
    return wl.random_bits(seed, kshape, dtype), wl.random_bits(seed + 1, vshape, dtype)


@pytest.mark.parametrize("dtype,Hkv,D", [("bf16", 2, 256), ("bf16", 8, 128), ("f32", 1, 64),
                                         ("bf16", 32, 256)])
def test_copy_blocks_bit_exact(dtype, Hkv, D):
    NB = 40
    kp0, vp0 = random_pools(900 + D + Hkv, NB, Hkv, D, dtype)
    src = [3, 7, 7, 11, 5, 2, -1, 9]
    dst = [20, 21, 22, 23, 5, 99, 30, 31]  # (5, 5) and the out-of-range ids are skipped
    banner("copy_blocks", dtype, Hkv, D)
    kp, vp = dev(kp0, dtype), dev(vp0, dtype)
    pkv.paged_kv_copy_blocks(i32(src), i32(dst), kp, vp)
    torch.cuda.synchronize()
    kr, vr = oracle.copy_blocks(src, dst, kp0, vp0)
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)


def test_copy_blocks_many_pairs():
    """A tick's worth of copies at once: 512 pairs over a 2048-block pool."""
    NB, Hkv, D = 2048, 2, 256
    kp0, vp0 = random_pools(950, NB, Hkv, D, "bf16")
    perm = np.random.default_rng(951).permutation(NB)
    src, dst = perm[:512], perm[512:1024]
    banner("copy_blocks 512 pairs")
    kp, vp = dev(kp0, "bf16"), dev(vp0, "bf16")
    pkv.paged_kv_copy_blocks(i32(src), i32(dst), kp, vp)
    torch.cuda.synchronize()
    kr, vr = oracle.copy_blocks(src, dst, kp0, vp0)
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)


@pytest.mark.parametrize("D", [128, 256])
def test_copy_on_write_then_decode_tick(D):
    """Sequences A and B share a 36-token prefix (blocks 0 and 1 full, block 2
    holding 4 tokens).  In one tick each appends its own token 36 into its
    logical block 2: the allocator gives B a private copy of that block
    first (one copy), A keeps the original.  Pools and outputs must match the
    oracle's copy then tick, and the shared full blocks stay shared."""
    Hq, Hkv, NB, dtype = 8, 2, 12, "bf16"
    kp0, vp0 = random_pools(960 + D, NB, Hkv, D, dtype)
    alloc = pkv.BlockAllocator(NB)
    row_a = alloc.alloc(3)
    alloc.share(row_a)
    row_b = row_a.copy()
    src_b, dst_b = alloc.prepare_write(row_b, 2, 2)
    src_a, dst_a = alloc.prepare_write(row_a, 2, 2)
    assert src_b.size == 1 and src_a.size == 0 and row_b[2] != row_a[2]
    assert alloc.refcount(int(row_a[0])) == 2 and alloc.refcount(int(row_a[2])) == 1

    tables = np.stack([row_a, row_b]).astype(np.int32)
    lens = np.array([37, 37], dtype=np.int32)
    q = wl.random_bits(970 + D, (2, Hq, D), dtype)
    kn = wl.random_bits(971 + D, (2, Hkv, D), dtype)
    vn = wl.random_bits(972 + D, (2, Hkv, D), dtype)
    scale = 1.0 / np.sqrt(D)
    banner("copy-on-write tick", D)

    kp, vp = dev(kp0, dtype), dev(vp0, dtype)
    pkv.paged_kv_copy_blocks(i32(src_b), i32(dst_b), kp, vp)
    qd = dev(q, dtype)
    out = torch.empty_like(qd)
    lse = torch.empty((2, Hq), dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_append(out, qd, dev(kn, dtype), dev(vn, dtype), kp, vp, i32(tables),
                                 i32(lens), 37, scale, 0.0, 0, lse=lse)
    torch.cuda.synchronize()

    kr, vr = oracle.copy_blocks(src_b, dst_b, kp0, vp0)
    ref, ref_lse, kr, vr = oracle.decode_append(q, kn, vn, kr, vr, tables, lens, scale,
                                                dtype=dtype)
    assert np.array_equal(pkv.to_bits(kp), kr) and np.array_equal(pkv.to_bits(vp), vr)
    check_close(as_f64(out), ref, dtype, "copy-on-write tick")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, "copy-on-write tick")
    # A's original block 2 kept its first 4 tokens and got A's token; B's copy
    # has the same first 4 tokens and B's token
    X = 8
    a2, b2 = int(row_a[2]), int(row_b[2])
    kb = pkv.to_bits(kp)
    assert np.array_equal(kb[a2, :, :, :4], kb[b2, :, :, :4])
    assert np.array_equal(kb[a2, :, :, 4, :], kn[0].reshape(Hkv, D // X, X))
    assert np.array_equal(kb[b2, :, :, 4, :], kn[1].reshape(Hkv, D // X, X))
