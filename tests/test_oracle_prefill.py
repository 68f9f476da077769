"""Pins for the oracle's chunked-prefill attention (CPU only).

``oracle.attention.prefill_attention`` is tied to things other than itself:
the scalar brute force of decode attention at context length p + 1 for the
row of position p (flat-index reads, ``math.fsum``), the decode oracle for
one-token chunks, causality (values after p never change row p, values at p
do), the first token of a prompt returning V_0, and a chunk that begins a
prompt (no history) reading only its own tokens.  Planted mistakes in the
oracle (off-by-one causal limits, positions counted from the wrong end)
fail these pins.
"""
import numpy as np
import pytest

import oracle.attention as att
import oracle.pool as pool


def _case(rng, lens, chunks, Hq=4, Hkv=2, d=8, bs=4, nb=40):
    """Tiny paged batch with a chunk of the newest chunks[s] tokens per sequence."""
    k, v = pool.new_pools(nb, Hkv, d, bs, np.float32)
    perm = rng.permutation(nb)
    maxb = max(1, max(-(-L // bs) for L in lens))
    tables = np.full((len(lens), maxb), -1, np.int64)
    used = 0
    for s, L in enumerate(lens):
        n = -(-L // bs)
        tables[s, :n] = perm[used:used + n]
        used += n
        kt = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        vt = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        pool.append(k, v, kt, vt, [int(tables[s, t // bs]) * bs + t % bs for t in range(L)])
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), Hq, d)).astype(np.float32)
    return q, k, v, tables, np.array(lens), qs


def _rows(lens, qs):
    """(row, sequence, position) of every query row."""
    out = []
    for s, L in enumerate(lens):
        C = int(qs[s + 1] - qs[s])
        out += [(int(qs[s]) + i, s, int(L) - C + i) for i in range(C)]
    return out


def test_rows_equal_decode_bruteforce_at_their_position():
    rng = np.random.default_rng(3)
    lens, chunks = [9, 5, 13, 1], [4, 5, 7, 1]
    q, k, v, t, L, qs = _case(rng, lens, chunks)
    got = att.prefill_attention(q, k, v, t, L, qs)
    for row, s, p in _rows(lens, qs):
        ref = att.decode_attention_bruteforce(q[row:row + 1], k, v, t[s:s + 1], [p + 1])[0]
        np.testing.assert_allclose(got[row], ref, rtol=0, atol=1e-13)


def test_one_token_chunks_equal_decode():
    rng = np.random.default_rng(4)
    lens = [7, 12, 3]
    q, k, v, t, L, qs = _case(rng, lens, [1, 1, 1])
    assert np.array_equal(att.prefill_attention(q, k, v, t, L, qs), att.decode_attention(q, k, v, t, L))


def test_causality():
    rng = np.random.default_rng(5)
    lens, chunks = [11], [6]
    q, k, v, t, L, qs = _case(rng, lens, chunks)
    base = att.prefill_attention(q, k, v, t, L, qs)
    bs = k.shape[3]
    for p_change in range(5, 11):  # change the K/V of one position
        k2, v2 = k.copy(), v.copy()
        b, o = int(t[0, p_change // bs]), p_change % bs
        k2[b, :, :, o, :] += 3.0
        v2[b, :, :, o] -= 2.0
        out = att.prefill_attention(q, k2, v2, t, L, qs)
        for row, _, p in _rows(lens, qs):
            if p < p_change:
                assert np.array_equal(out[row], base[row]), (p, p_change)
            else:
                assert not np.allclose(out[row], base[row]), (p, p_change)


def test_first_prompt_token_returns_v0_and_no_history_reads_only_the_chunk():
    rng = np.random.default_rng(6)
    lens, chunks = [6, 9], [6, 3]
    q, k, v, t, L, qs = _case(rng, lens, chunks)
    got = att.prefill_attention(q, k, v, t, L, qs)
    k0, v0 = pool.gather(k, v, t[0], 6)
    G = 2
    for h in range(4):
        np.testing.assert_array_equal(got[0, h], v0[0, h // G].astype(np.float64))


def test_rejects_bad_offsets():
    rng = np.random.default_rng(7)
    q, k, v, t, L, qs = _case(rng, [3], [3])
    with pytest.raises(ValueError):
        att.prefill_attention(q, k, v, t, L, np.array([0, 4]))  # more rows than q has
    with pytest.raises(ValueError):
        att.prefill_attention(q[:3], k, v, t, np.array([2]), np.array([0, 3]))  # chunk longer than context
    zero = att.prefill_attention(q[:0], k, v, t, L, np.array([0, 0]))
    assert zero.shape == (0, 4, 8)


# ---------------------------------------------------------------- mutants
def _prefill_causal_off_by_one(q, k_pool, v_pool, block_tables, context_lens, query_start, scale=None):
    q64 = pool.to_f64(q)
    out = np.zeros(q64.shape)
    d = q64.shape[-1]
    for s in range(len(query_start) - 1):
        L, C = int(context_lens[s]), int(query_start[s + 1] - query_start[s])
        ks, vs = pool.gather(k_pool, v_pool, block_tables[s], L)
        for i in range(C):
            p = L - C + i
            out[query_start[s] + i] = att.dense_attention(q64[query_start[s] + i], pool.to_f64(ks)[:p],
                                                          pool.to_f64(vs)[:p], 1 / np.sqrt(d)) if p else 0
    return out


def _prefill_positions_from_start(q, k_pool, v_pool, block_tables, context_lens, query_start, scale=None):
    q64 = pool.to_f64(q)
    out = np.zeros(q64.shape)
    d = q64.shape[-1]
    for s in range(len(query_start) - 1):
        L, C = int(context_lens[s]), int(query_start[s + 1] - query_start[s])
        ks, vs = pool.gather(k_pool, v_pool, block_tables[s], L)
        for i in range(C):
            p = i  # wrong: the chunk is the newest tokens, not the first ones
            out[query_start[s] + i] = att.dense_attention(q64[query_start[s] + i], pool.to_f64(ks)[:p + 1],
                                                          pool.to_f64(vs)[:p + 1], 1 / np.sqrt(d))
    return out


@pytest.mark.parametrize("mutant", [_prefill_causal_off_by_one, _prefill_positions_from_start],
                         ids=["causal-off-by-one", "positions-from-start"])
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(att, "prefill_attention", mutant)
    with pytest.raises(AssertionError):
        test_rows_equal_decode_bruteforce_at_their_position()
