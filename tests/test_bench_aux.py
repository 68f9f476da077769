"""Host-side accounting in bench.py (CPU only): the algorithmic byte and flop
counts behind the roofline figures, and the slot-waste comparison of paging
against a contiguous max-length reservation."""
import sys
import os

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_decode_bytes_70b_32k_closed_form():
    # 16 sequences of 32773 tokens (the first timed step), 64/8 heads, d 128, bs 16, bf16
    lens = [32773] * 16
    kv = 16 * 32773 * 8 * 128 * 2 * 2
    assert bench.decode_kv_bytes(lens, 8, 128, 2) == kv
    qo = 2 * 16 * 64 * 128 * 2
    tables = 4 * 16 * 2049  # ceil(32773 / 16) entries per sequence
    assert bench.decode_algorithmic_bytes(lens, 64, 8, 128, 16, 2) == kv + qo + tables + 4 * 16 == 2148466816


def test_append_bytes_count_one_row_per_nonempty_sequence():
    # each non-empty sequence's new K and V rows: read once from k_new/v_new, written once into the pool
    # 70B step: 16 x 8 x 128 bf16 = 32 KiB of K rows and 32 KiB of V rows, each read and written: 128 KiB
    assert bench.append_algorithmic_bytes([32773] * 16, 8, 128, 2) == 16 * 8 * 128 * 2 * 2 * 2 == 131072
    assert bench.append_algorithmic_bytes([5, 0, 1], 2, 64, 4) == 2 * (2 * 64 * 4) * 2 * 2
    assert bench.append_algorithmic_bytes([], 8, 128, 2) == 0


def test_prefill_flops_equal_brute_force():
    lens, chunks = [7, 20, 5], [3, 20, 1]
    brute = 0
    for L, C in zip(lens, chunks):
        for p in range(L - C, L):  # token at position p reads keys 0..p
            brute += 4 * 8 * 64 * (p + 1)
    assert bench.prefill_flops(lens, chunks, 8, 64) == brute


def test_paging_waste():
    w = bench.paging_waste([17, 33, 64, 100], 16, 112)
    assert w["paged_slots"] == (2 + 3 + 4 + 7) * 16 and w["tokens"] == 214
    assert abs(w["paged_waste"] - 42 / 256) < 1e-5 and abs(w["reserved_waste"] - (448 - 214) / 448) < 1e-5
    # whole-block paging wastes fewer than block_size slots per sequence
    lens = [1, 16, 17, 1000, 4095]
    w = bench.paging_waste(lens, 32, 4096)
    assert w["paged_slots"] - w["tokens"] < 32 * len(lens)
    assert bench.paging_waste([16, 32], 16, 32)["paged_waste"] == 0.0


def test_more_than_one_gpu_is_refused():
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_decode_tile_ids_are_the_tiles_a_decode_call_reads():
    """The tile-read ceiling streams exactly the (block, kv head) tiles of the
    call: every block of each sequence's first ceil(L / bs) table entries,
    for every kv head, head by head; empty sequences add nothing."""
    import numpy as np

    rng = np.random.default_rng(5)
    bs, hkv, width = 16, 4, 9
    lens = np.array([1, 0, 16, 17, 140, 33], dtype=np.int32)
    tables = rng.permutation(200)[: len(lens) * width].reshape(len(lens), width).astype(np.int32)
    ids = bench.decode_tile_ids(tables, lens, bs, hkv)
    nb = [-(-int(L) // bs) for L in lens]
    per_head = sum(nb)
    assert ids.dtype == np.int32 and ids.size == hkv * per_head
    rows = np.concatenate([tables[s, :nb[s]] for s in range(len(lens))])
    for g in range(hkv):
        seg = ids[g * per_head:(g + 1) * per_head].astype(np.int64)
        assert np.array_equal(seg % hkv, np.full(per_head, g))
        assert np.array_equal(seg // hkv, rows)
    assert bench.decode_tile_ids(tables[:2], np.array([0, 0]), bs, hkv).size == 0
