"""Pins for the oracle's pool format, append scatter and block copy (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_layout_matches_hand_written_fixture():
    with open(os.path.join(GOLDEN, "pool_layout_tiny.json")) as f:
        fx = json.load(f)
    k, v = pool.new_pools(fx["num_blocks"], fx["num_kv_heads"], fx["head_dim"], fx["block_size"], np.float32)
    H, d = fx["num_kv_heads"], fx["head_dim"]
    kn = np.array([t["k"] for t in fx["tokens"]], np.float32).reshape(-1, H, d)
    vn = np.array([t["v"] for t in fx["tokens"]], np.float32).reshape(-1, H, d)
    pool.append(k, v, kn, vn, [t["slot"] for t in fx["tokens"]])
    assert k.reshape(-1).tolist() == fx["k_flat"]
    assert v.reshape(-1).tolist() == fx["v_flat"]


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
@pytest.mark.parametrize("bs", [16, 32])
def test_append_gather_round_trip(dtype, bs):
    rng = np.random.default_rng(7)
    H, d, nb = 3, 64, 40
    k, v = pool.new_pools(nb, H, d, bs, dtype)
    perm = rng.permutation(nb)
    L = 5 * bs + 7  # several blocks plus a ragged tail
    if dtype == np.uint16:
        kt = rng.integers(0, 1 << 16, size=(L, H, d)).astype(np.uint16)
        vt = rng.integers(0, 1 << 16, size=(L, H, d)).astype(np.uint16)
    else:
        kt = rng.standard_normal((L, H, d)).astype(np.float32)
        vt = rng.standard_normal((L, H, d)).astype(np.float32)
    table = perm[: -(-L // bs)]
    slots = [int(table[t // bs]) * bs + t % bs for t in range(L)]
    order = rng.permutation(L)  # write order must not matter
    pool.append(k, v, kt[order], vt[order], np.array(slots)[order])
    kg, vg = pool.gather(k, v, table, L)
    assert kg.dtype == kt.dtype and np.array_equal(kg.view(np.uint8), kt.view(np.uint8))
    assert np.array_equal(vg.view(np.uint8), vt.view(np.uint8))


def test_negative_slot_is_skipped():
    k, v = pool.new_pools(2, 1, 8, 2, np.float32)
    pool.append(k, v, np.ones((2, 1, 8), np.float32), np.ones((2, 1, 8), np.float32), [-1, 1])
    assert k.sum() == 8 and v.sum() == 8
    assert k[0, 0, :, 1, :].sum() == 8


def test_copy_blocks_duplicates_and_leaves_source():
    rng = np.random.default_rng(3)
    k, v = pool.new_pools(6, 2, 16, 16, np.uint16)
    k[:] = rng.integers(0, 1 << 16, size=k.shape)
    v[:] = rng.integers(0, 1 << 16, size=v.shape)
    k0, v0 = k.copy(), v.copy()
    pool.copy_blocks(k, v, [(1, 4), (2, 5)])
    assert np.array_equal(k[4], k0[1]) and np.array_equal(v[5], v0[2])
    for b in (0, 1, 2, 3):  # everything but the destinations untouched
        assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])


def test_bf16_decoding_textbook_values():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x0001], np.uint16)
    got = pool.to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 0.0 and np.signbit(got[4]) and np.isinf(got[5])
    assert got[6] == 2.0 ** -133  # smallest bf16 subnormal


def test_gather_rejects_short_table():
    k, v = pool.new_pools(4, 1, 8, 4, np.float32)
    with pytest.raises(IndexError):
        pool.gather(k, v, [0], 5)
