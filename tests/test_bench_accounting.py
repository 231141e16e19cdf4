"""The bench's algorithmic work counts (the numerators of every rate it
reports) against closed forms worked out from the workload definitions:
the long-context decode (8 x 32768 tokens, 4 kv heads, D 128, bf16), the
sliding-window decode (window 512 over contexts of 2048-8192), the chunked
prefill (8 x (2048 cached + 512 new), 8 query heads, D 256, causal) and the
append of its chunk, and the decode tick (the decode plus its appended rows).
CPU only: no kernel runs here."""
import bench
from block_paged_kv_append_amd import workloads as wl


def test_long_context_decode_bytes():
    c = wl.long_context_splitk()
    kv = 8 * 32768 * 4 * 128 * 2 * 2            # K and V, once per kv head
    q_out = 2 * 8 * 32 * 128 * 2                # q read, out written
    meta = 4 * (8 + 8 * (32768 // 16))          # lengths, one table entry per block
    assert bench.decode_bytes(c) == kv + q_out + meta == 537_067_552


def test_sliding_window_decode_bytes():
    c = wl.sliding_window_decode()
    lens = [int(x) for x in c.context_lens]
    assert min(lens) >= 2048                    # every sequence sees a full window
    kv = 32 * 512 * 2 * 256 * 2 * 2
    blocks = sum((L - 1) // 16 - (L - 512) // 16 + 1 for L in lens)  # blocks the window touches
    assert bench.decode_bytes(c) == kv + 2 * 32 * 8 * 256 * 2 + 4 * (32 + blocks)
    assert kv == 33_554_432


def test_tick_bytes_add_the_appended_rows():
    c = wl.gemma_decode()
    assert bench.tick_bytes(c) - bench.decode_bytes(c) == 2 * 2 * 32 * 2 * 256 * 2


def test_chunked_prefill_flops_and_append_bytes():
    c = wl.chunked_prefill_shared_prefix()
    # query j of the chunk sits at position 2048 + j and sees keys 0 .. 2048 + j
    pairs_per_seq_head = sum(2048 + j + 1 for j in range(512))
    assert bench.prefill_flops(c) == 4.0 * 256 * 8 * 8 * pairs_per_seq_head == 77_326_188_544.0
    assert bench.append_bytes(4096, 2, 256, 2) == 2 * (2 * 4096 * 2 * 256 * 2) + 4 * 4096
