"""The measurement probes that give the bench its measured ceilings read and
compute what they claim: the streaming read and the tile read fold every
word they read into their workgroup's sink word (checked against the same
fold on the host), and the matrix-core probe's result is the same in every
workgroup and zero without products.  The ceilings they give are those of
the bandwidth-bound decode ("PagedAttention" (robocikowo.com), Złożoność
obliczeniowa) and the matrix-core-bound chunked prefill ("PagedAttention et
RadixAttention : parlons de KV Cache", the part on the two independent
problems)."""
import numpy as np
import pytest
import torch

from helpers import say

pytestmark = pytest.mark.gpu

THREADS = 256  # the probes' workgroup size (4 waves)


def _xor_fold(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32).ravel(), initial=np.uint32(0)))


@pytest.mark.parametrize("tile_bytes,num_tiles,max_tiles,sink_words", [
    (4096, 301, 64, 4096),   # repeats, odd count, several waves per workgroup share
    (1024, 1000, 97, 8),     # grid capped by the sink: long shares per wave
    (2048, 7, 7, 64),        # fewer tiles than waves
])
def test_tile_read_folds_the_listed_tiles(tile_bytes, num_tiles, max_tiles, sink_words):
    import paged_kv_cache_230_amd as pkv

    g = torch.Generator().manual_seed(tile_bytes + num_tiles)
    words_per_tile = tile_bytes // 4
    pool_h = torch.randint(-2**31, 2**31 - 1, (max_tiles * words_per_tile,), generator=g, dtype=torch.int64)
    pool_h = pool_h.to(torch.int32)
    ids_h = torch.randint(-3, max_tiles + 3, (num_tiles,), generator=g, dtype=torch.int32)  # some out of range
    pool = pool_h.cuda()
    ids = ids_h.cuda()
    sink = torch.zeros(sink_words, dtype=torch.int32, device="cuda")
    pkv.tile_read(pool, tile_bytes, ids, sink)
    torch.cuda.synchronize()

    # The same partition on the host: grid = min(sink_words, workgroups for
    # two tiles per wave), each wave a contiguous share of the list, indices
    # clamped to the pool; a workgroup's word folds its four waves' tiles.
    waves_needed = -(-num_tiles // 2)
    grid = min(sink_words, -(-waves_needed // (THREADS // 64)))
    nwaves = grid * (THREADS // 64)
    tiles = pool_h.numpy().view(np.uint32).reshape(max_tiles, words_per_tile)
    clamped = np.clip(ids_h.numpy().astype(np.int64), 0, max_tiles - 1)
    want = np.zeros(grid, dtype=np.uint32)
    for wv in range(nwaves):
        t0, t1 = num_tiles * wv // nwaves, num_tiles * (wv + 1) // nwaves
        f = 0
        for t in range(t0, t1):
            f ^= _xor_fold(tiles[clamped[t]])
        want[wv // (THREADS // 64)] ^= np.uint32(f)
    got = sink.cpu().numpy().view(np.uint32)[:grid]
    say(f"  tile read: {num_tiles} tiles of {tile_bytes} B over {grid} workgroups")
    assert np.array_equal(got, want)


def test_stream_read_folds_the_buffer():
    import paged_kv_cache_230_amd as pkv

    g = torch.Generator().manual_seed(11)
    nbytes = 16 * 5000 + 16 * 37  # not a multiple of the workgroup's 4 KiB
    buf_h = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    pkv.stream_read(buf_h.cuda(), sink)
    torch.cuda.synchronize()
    # min(bytes / 4096, sink_words) workgroups, each a contiguous share of
    # the 16-byte chunks
    n = nbytes // 16
    grid = min(-(-n // THREADS), 64)
    chunks = buf_h.numpy().view(np.uint32).reshape(n, 4)
    want = np.array([_xor_fold(chunks[n * b // grid:n * (b + 1) // grid]) for b in range(grid)], dtype=np.uint32)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32)[:grid], want)


def test_mfma_rate_is_the_same_in_every_workgroup():
    import paged_kv_cache_230_amd as pkv

    wg = 6
    sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = pkv.mfma_rate(sink, wg, 3)
    torch.cuda.synchronize()
    assert flops == wg * 8 * 3 * 16 * 32768
    s = sink.cpu().view(wg, 512)
    assert torch.isfinite(s).all()
    assert torch.equal(s, s[:1].expand_as(s))  # every workgroup computes the same products
    assert (s.abs() > 0).any()
    pkv.mfma_rate(sink, wg, 0)
    torch.cuda.synchronize()
    assert torch.equal(sink.cpu(), torch.zeros(wg * 512))
