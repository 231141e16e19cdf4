"""Host-only checks of the refcounted block allocator (pkv_block_allocator):
no GPU needed.  Every operation is mirrored in a plain Python model of
refcounts written here, and random operation sequences must keep the two in
agreement, with every error leaving the allocator unchanged."""
import os

import numpy as np
import pytest

import block_paged_kv_append_amd as pkv

pytestmark = pytest.mark.skipif(not os.path.exists(pkv.LIB_PATH),
                                reason="libpkv.so not built (run __graft_entry__.build())")


def test_alloc_hands_out_distinct_ids_in_order_and_runs_out():
    a = pkv.BlockAllocator(6)
    assert a.num_free() == 6
    ids = a.alloc(4)
    assert ids.tolist() == [0, 1, 2, 3]
    assert [a.refcount(i) for i in range(6)] == [1, 1, 1, 1, 0, 0]
    with pytest.raises(pkv.PkvError) as e:
        a.alloc(3)
    assert e.value.code == -5 and a.num_free() == 2  # all or nothing
    a.release([1])
    assert a.num_free() == 3 and a.refcount(1) == 0
    assert a.alloc(1).tolist() == [1]  # the freed id comes back first
    assert a.refcount(99) == -1 and a.refcount(-1) == -1


def test_share_release_and_errors_leave_state_unchanged():
    a = pkv.BlockAllocator(4)
    ids = a.alloc(2)
    a.share(ids)
    a.share(ids[:1])
    assert [a.refcount(i) for i in ids] == [3, 2]
    with pytest.raises(pkv.PkvError):
        a.share([0, 3])  # 3 is free: nothing changes
    assert [a.refcount(i) for i in ids] == [3, 2]
    with pytest.raises(pkv.PkvError):
        a.release([1, 1, 1])  # held twice only
    assert a.refcount(1) == 2
    a.release([1, 1])
    assert a.refcount(1) == 0 and a.num_free() == 3


def test_prepare_write_copies_only_shared_blocks():
    a = pkv.BlockAllocator(10)
    prefix = a.alloc(3)                       # sequence A: blocks 0, 1, 2
    row_a = np.concatenate([prefix, a.alloc(1)]).astype(np.int32)
    a.share(prefix)                           # sequence B forks A's prefix
    row_b = np.concatenate([prefix, a.alloc(1)]).astype(np.int32)
    before = row_b.copy()
    src, dst = a.prepare_write(row_b, 2, 3)   # B writes into its logical blocks 2..3
    assert src.tolist() == [int(prefix[2])]   # block 2 is shared, block 3 is B's own
    assert row_b[2] == dst[0] and row_b[3] == before[3] and row_b[:2].tolist() == before[:2].tolist()
    assert a.refcount(int(prefix[2])) == 1 and a.refcount(int(dst[0])) == 1
    assert row_a.tolist() == [0, 1, 2, 3]      # A's table is untouched
    # nothing shared any more in that range: no copies
    s2, d2 = a.prepare_write(row_b, 2, 3)
    assert s2.size == 0 and d2.size == 0


def test_prepare_write_is_all_or_nothing_when_short_of_blocks():
    a = pkv.BlockAllocator(4)
    row = a.alloc(2)
    a.share(row)
    a.alloc(2)  # pool now empty
    r = row.astype(np.int32).copy()
    with pytest.raises(pkv.PkvError) as e:
        a.prepare_write(r, 0, 1)
    assert e.value.code == -5
    assert r.tolist() == row.tolist() and [a.refcount(int(i)) for i in row] == [2, 2]
    with pytest.raises(pkv.PkvError):
        a.prepare_write(np.array([0, 7], dtype=np.int32), 0, 1)  # 7 out of range


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_a_refcount_model(seed):
    rng = np.random.default_rng(seed)
    NB = 24
    a = pkv.BlockAllocator(NB)
    ref = [0] * NB
    tables = []  # python lists of ids held by each "sequence"
    for step in range(400):
        op = rng.integers(0, 5)
        if op == 0:  # new sequence
            n = int(rng.integers(1, 5))
            if n <= ref.count(0):
                ids = a.alloc(n).tolist()
                assert all(ref[i] == 0 for i in ids) and len(set(ids)) == n
                for i in ids:
                    ref[i] = 1
                tables.append(ids)
            else:
                with pytest.raises(pkv.PkvError):
                    a.alloc(n)
        elif op == 1 and tables:  # fork a prefix of a sequence
            t = tables[int(rng.integers(len(tables)))]
            k = int(rng.integers(1, len(t) + 1))
            a.share(t[:k])
            for i in t[:k]:
                ref[i] += 1
            tables.append(list(t[:k]))
        elif op == 2 and tables:  # a sequence ends
            t = tables.pop(int(rng.integers(len(tables))))
            a.release(t)
            for i in t:
                ref[i] -= 1
        elif op == 3 and tables:  # a sequence writes into a range of its blocks
            t = tables[int(rng.integers(len(tables)))]
            lo = int(rng.integers(len(t)))
            hi = int(rng.integers(lo, len(t)))
            row = np.array(t, dtype=np.int32)
            need = sum(ref[i] > 1 for i in t[lo:hi + 1])
            if need <= ref.count(0):
                src, dst = a.prepare_write(row, lo, hi)
                assert len(src) == need
                for s_, d_ in zip(src.tolist(), dst.tolist()):
                    assert ref[d_] == 0 and ref[s_] > 1
                    ref[s_] -= 1
                    ref[d_] = 1
                t[:] = row.tolist()
                assert all(ref[i] == 1 for i in t[lo:hi + 1])
            else:
                with pytest.raises(pkv.PkvError):
                    a.prepare_write(row, lo, hi)
                assert row.tolist() == t
        # the model and the allocator agree after every step
        assert [a.refcount(i) for i in range(NB)] == ref
        assert a.num_free() == ref.count(0)
        held = {}
        for t in tables:
            for i in t:
                held[i] = held.get(i, 0) + 1
        assert all(ref[i] == held.get(i, 0) for i in range(NB))
