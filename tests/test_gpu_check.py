"""pkv_check_paged_metadata on the device: valid metadata of the bench
workloads reports nothing; each planted breach of the contract (a length out
of range, a block id out of the pool in an entry the sequence reads, a slot
out of the pool, a repeated slot) reports its own flag and only that; entries
past a sequence's length are not checked.  The expected flags come from the
contract restated in numpy below."""
import numpy as np
import pytest
import torch

import block_paged_kv_append_amd as pkv
from block_paged_kv_append_amd import workloads as wl
from tests.gpu_common import i32

pytestmark = pytest.mark.gpu


def expected_flags(block_tables, context_lens, num_blocks, slot_mapping):
    bt = np.asarray(block_tables, dtype=np.int64).reshape(len(context_lens), -1)
    span = bt.shape[1] * 16
    f = 0
    for b, L in enumerate(np.asarray(context_lens, dtype=np.int64)):
        if L < 0 or L > span:
            f |= pkv.CHECK_BAD_CONTEXT_LEN
        Lc = min(max(L, 0), span)
        read = bt[b, :(Lc + 15) // 16]
        if ((read < 0) | (read >= num_blocks)).any():
            f |= pkv.CHECK_BAD_BLOCK_ID
    s = np.asarray(slot_mapping, dtype=np.int64)
    s = s[s >= 0]
    if (s >= num_blocks * 16).any():
        f |= pkv.CHECK_BAD_SLOT
    s = s[s < num_blocks * 16]
    if len(np.unique(s)) != len(s):
        f |= pkv.CHECK_DUPLICATE_SLOT
    return f


def run(bt, cl, nb, sm):
    got = pkv.check_paged_metadata(nb, i32(bt) if bt is not None else None,
                                   i32(cl) if cl is not None else None,
                                   i32(sm) if sm is not None else None)
    return got


def test_bench_workloads_are_valid():
    for c in (wl.gemma_decode(), wl.sliding_window_decode()):
        print("case:", c.name, flush=True)
        assert run(c.block_tables, c.context_lens, c.num_blocks, None) == 0
    p = wl.chunked_prefill_shared_prefix()
    print("case:", p.name, flush=True)
    assert run(p.block_tables, p.context_lens, p.num_blocks, p.slot_mapping) == 0


def test_each_breach_sets_its_flag():
    rng = np.random.default_rng(5)
    B, MB, NB = 6, 9, 40
    bt = rng.integers(0, NB, size=(B, MB)).astype(np.int32)
    cl = np.array([0, 1, 16, 17, 100, MB * 16], dtype=np.int32)
    sm = rng.permutation(NB * 16)[:50].astype(np.int32)
    sm[[3, 11]] = -1  # skipped rows
    cases = {"valid": (bt, cl, sm)}
    b2 = bt.copy(); b2[4, 6] = NB                     # entry 6 of a 100-token sequence is read
    cases["block id past the pool"] = (b2, cl, sm)
    b3 = bt.copy(); b3[3, 1] = -7                      # entry 1 of a 17-token sequence is read
    cases["negative block id"] = (b3, cl, sm)
    b4 = bt.copy(); b4[2, 1] = NB + 5; b4[0, :] = -1   # past the 16-token length / empty sequence
    cases["entries past the length"] = (b4, cl, sm)
    c5 = cl.copy(); c5[1] = MB * 16 + 1
    cases["length past the table"] = (bt, c5, sm)
    c6 = cl.copy(); c6[0] = -2
    cases["negative length"] = (bt, c6, sm)
    s7 = sm.copy(); s7[7] = NB * 16
    cases["slot past the pool"] = (bt, cl, s7)
    s8 = sm.copy(); s8[49] = s8[0]
    cases["repeated slot"] = (bt, cl, s8)
    s9 = sm.copy(); s9[:] = -1
    cases["all rows skipped"] = (bt, cl, s9)
    b10, c10, s10 = b2.copy(), c5.copy(), s8.copy(); s10[7] = NB * 16 + 3
    cases["every breach"] = (b10, c10, s10)
    seen = set()
    for name, (b, c, s) in cases.items():
        print("case:", name, flush=True)
        want = expected_flags(b, c, NB, s)
        assert run(b, c, NB, s) == want, name
        seen.add(want)
    assert {0, pkv.CHECK_BAD_BLOCK_ID, pkv.CHECK_BAD_CONTEXT_LEN, pkv.CHECK_BAD_SLOT,
            pkv.CHECK_DUPLICATE_SLOT, 15} <= seen


def test_large_slot_mapping_and_tables():
    """Thousands of table entries and slots (many workgroups): one repeated
    slot at the two ends, and one bad block id in the last entry of the last
    sequence (read only if that sequence is long enough), are found."""
    p = wl.chunked_prefill_shared_prefix()
    sm = np.asarray(p.slot_mapping, dtype=np.int32).copy()
    assert run(None, None, p.num_blocks, sm) == 0
    sm[-1] = sm[0]
    assert run(None, None, p.num_blocks, sm) == pkv.CHECK_DUPLICATE_SLOT
    c = wl.gemma_decode()
    bt = np.asarray(c.block_tables, dtype=np.int32).copy()
    last = (int(c.context_lens[-1]) + 15) // 16 - 1  # the last entry the sequence reads
    bt[-1, last] = c.num_blocks
    want = expected_flags(bt, c.context_lens, c.num_blocks, [])
    assert want == pkv.CHECK_BAD_BLOCK_ID
    assert run(bt, c.context_lens, c.num_blocks, None) == want
    bt[-1, last] = 0
    bt[-1, last + 1:] = -1  # entries past the length are not checked
    assert run(bt, c.context_lens, c.num_blocks, None) == 0


def test_empty_check_reports_nothing():
    assert pkv.check_paged_metadata(4) == 0
    torch.cuda.synchronize()


def test_hbm_read_probe_reads_every_word_once():
    """The read probe folds every 32-bit word of the buffer into the
    workgroups' words by XOR: their XOR is the XOR of the whole buffer (each
    word read exactly once), for sizes with and without a ragged tail."""
    for nbytes, wgs in ((1 << 20, 64), (3 * 4096 + 48, 7), (16, 1)):
        print("\n[case] read probe", nbytes, wgs, flush=True)
        host = np.random.default_rng(nbytes).integers(0, 2**32, size=nbytes // 4, dtype=np.uint64)
        host = host.astype(np.uint32)
        buf = torch.from_numpy(host.view(np.int32).copy()).cuda()
        out = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        pkv.hbm_read_probe(buf, out, num_wgs=wgs)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host)


def test_hbm_gather_probe_reads_each_listed_block_once():
    """The gather probe folds every 32-bit word of each listed block of K and V
    into the workgroups' words by XOR (blocks listed twice cancel, entries
    outside the pools read block 0); ragged ranges per workgroup."""
    rng = np.random.default_rng(5)
    nb, words = 37, 4096 // 4
    k = rng.integers(0, 2**32, size=(nb, words), dtype=np.uint64).astype(np.uint32)
    v = rng.integers(0, 2**32, size=(nb, words), dtype=np.uint64).astype(np.uint32)
    order = rng.integers(0, nb, size=101).astype(np.int32)
    order[[3, 50]] = [nb + 5, -2]  # outside the pools: block 0
    kd = torch.from_numpy(k.view(np.int32).copy()).cuda()
    vd = torch.from_numpy(v.view(np.int32).copy()).cuda()
    for wgs in (1, 7, 64):
        print("\n[case] gather probe", wgs, flush=True)
        out = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        pkv.hbm_gather_probe(kd, vd, torch.from_numpy(order).cuda(), out, num_wgs=wgs)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        ids = np.where((order >= 0) & (order < nb), order, 0)
        want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(k[ids], axis=1) ^
                                     np.bitwise_xor.reduce(v[ids], axis=1))
        assert got == want


def test_mfma_rate_probe_records_every_workgroup():
    """The matrix-core rate probe writes, per workgroup, shader-clock and
    100 MHz counter pairs that advance over the loop; the cycles per product
    are at least the 32 a 32x32x16 bf16 product takes (8 passes of 4 cycles)
    and the implied clock lies in the part's range."""
    wgs, iters = 8, 2000
    print("\n[case] matrix-core rate probe", wgs, iters, flush=True)
    stamps = torch.zeros(4 * wgs, dtype=torch.int64, device="cuda")
    pkv.mfma_rate_probe(stamps, iters, num_wgs=wgs)
    torch.cuda.synchronize()
    s = stamps.cpu().numpy().reshape(wgs, 4).astype(np.float64)
    cycles, ticks = s[:, 1] - s[:, 0], s[:, 3] - s[:, 2]
    assert np.all(cycles > 0) and np.all(ticks > 0)
    per_product = cycles / (iters * 8)
    assert np.all(per_product >= 32) and np.all(per_product < 200), per_product
    mhz = cycles / ticks * 100.0
    assert np.all((mhz > 500) & (mhz < 3000)), mhz

