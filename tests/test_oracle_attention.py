"""Pins for the oracle's decode attention (CPU only).

Each pin ties ``oracle.attention`` to something other than itself: a scalar
brute force, a closed form, or an invariant the pages fix (paging does not
change the result).  ``test_pins_catch_planted_mistakes`` plants plausible
mistakes in the oracle and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle.attention as att
import oracle.pool as pool


def _paged_case(rng, S=3, Hq=4, Hkv=2, d=8, bs=4, lens=(1, 4, 9), nb=16, dtype=np.float32, kv_std=1.0):
    """Random tiny paged batch: pools, tables (random physical blocks) and the logical rows."""
    k, v = pool.new_pools(nb, Hkv, d, bs, dtype)
    perm = rng.permutation(nb)
    maxb = max(-(-L // bs) for L in lens)
    tables = np.full((S, maxb), -1, np.int64)
    logical = []
    used = 0
    for s, L in enumerate(lens):
        nblk = -(-L // bs)
        tables[s, :nblk] = perm[used : used + nblk]
        used += nblk
        kt = (rng.standard_normal((L, Hkv, d)) * kv_std).astype(np.float32)
        vt = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        slots = [int(tables[s, t // bs]) * bs + t % bs for t in range(L)]
        pool.append(k, v, kt, vt, slots)
        logical.append((kt.astype(np.float64), vt.astype(np.float64)))
    q = rng.standard_normal((S, Hq, d)).astype(np.float32)
    return q, k, v, tables, np.array(lens), logical


# ---------------------------------------------------------------- pins
def pin_bruteforce():
    rng = np.random.default_rng(11)
    q, k, v, tables, lens, _ = _paged_case(rng)
    a = att.decode_attention(q, k, v, tables, lens)
    b = att.decode_attention_bruteforce(q, k, v, tables, lens)
    return np.allclose(a, b, rtol=0, atol=1e-12)


def pin_single_token_returns_v0():
    rng = np.random.default_rng(12)
    q, k, v, tables, lens, logical = _paged_case(rng, S=1, lens=(1,))
    out = att.decode_attention(q, k, v, tables, lens)
    G = q.shape[1] // k.shape[1]
    want = np.stack([logical[0][1][0, h // G] for h in range(q.shape[1])])
    return np.array_equal(out[0], want)


def pin_zero_query_gives_mean():
    rng = np.random.default_rng(13)
    q, k, v, tables, lens, logical = _paged_case(rng, S=2, lens=(7, 13))
    q[:] = 0
    out = att.decode_attention(q, k, v, tables, lens)
    G = q.shape[1] // k.shape[1]
    ok = True
    for s in range(2):
        for h in range(q.shape[1]):
            want = logical[s][1][:, h // G].mean(axis=0)
            ok &= np.allclose(out[s, h], want, rtol=1e-13, atol=1e-14)
    return bool(ok)


def pin_equal_keys_give_mean():
    rng = np.random.default_rng(14)
    q, k, v, tables, lens, logical = _paged_case(rng, S=1, lens=(11,))
    # rebuild the cache with every key equal to the first one
    kt = np.repeat(logical[0][0][:1], 11, axis=0).astype(np.float32)
    vt = logical[0][1].astype(np.float32)
    bs = k.shape[3]
    slots = [int(tables[0, t // bs]) * bs + t % bs for t in range(11)]
    pool.append(k, v, kt, vt, slots)
    out = att.decode_attention(q, k, v, tables, lens)
    G = q.shape[1] // k.shape[1]
    return all(
        np.allclose(out[0, h], vt[:, h // G].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-14)
        for h in range(q.shape[1])
    )


def pin_constant_values():
    rng = np.random.default_rng(15)
    q, k, v, tables, lens, _ = _paged_case(rng, S=2, lens=(5, 10))
    c = np.arange(k.shape[1] * 8, dtype=np.float32).reshape(k.shape[1], 8) - 3.5  # per kv head
    v[:] = np.broadcast_to(c[None, :, :, None], v.shape)
    out = att.decode_attention(q, k, v, tables, lens)
    G = q.shape[1] // k.shape[1]
    return all(np.allclose(out[s, h], c[h // G], rtol=1e-14, atol=1e-14) for s in range(2) for h in range(q.shape[1]))


def pin_two_tokens_logistic():
    """out = V0 + sigmoid(z1 - z0) (V1 - V0), z_t = <q, k_t>/sqrt(d)."""
    d = 8
    k, v = pool.new_pools(2, 1, d, 4, np.float32)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, :] = [1, 2, 0, 0, -1, 0, 0, 0.5]
    k0 = np.array([0.5, 0, 1, 0, 0, 0, 2, 0], np.float32)
    k1 = np.array([1, 1, 0, 0, 1, 0, 0, 2], np.float32)
    v0 = np.arange(d, dtype=np.float32)
    v1 = -2.0 * np.arange(d, dtype=np.float32) + 1
    pool.append(k, v, np.stack([k0, k1])[:, None], np.stack([v0, v1])[:, None], [4, 5])
    out = att.decode_attention(q, k, v, np.array([[1]]), np.array([2]))
    z0 = (0.5 * 1) / math.sqrt(d)
    z1 = (1 + 2 - 1 + 1) / math.sqrt(d)
    w = 1.0 / (1.0 + math.exp(-(z1 - z0)))
    want = v0.astype(np.float64) + w * (v1.astype(np.float64) - v0.astype(np.float64))
    return np.allclose(out[0, 0], want, rtol=1e-14, atol=1e-14)


def pin_needle():
    rng = np.random.default_rng(16)
    d, L, bs = 16, 37, 16
    k, v = pool.new_pools(8, 1, d, bs, np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    kt = (rng.standard_normal((L, 1, d)) * 0.01).astype(np.float32)
    vt = rng.standard_normal((L, 1, d)).astype(np.float32)
    j = 23
    kt[j, 0] = 50.0 * q[0, 0]
    table = np.array([[5, 2, 7]])
    pool.append(k, v, kt, vt, [int(table[0, t // bs]) * bs + t % bs for t in range(L)])
    out = att.decode_attention(q, k, v, table, np.array([L]))
    return np.allclose(out[0, 0], vt[j, 0], atol=1e-6)


def pin_gqa_equals_replicated_mha():
    rng = np.random.default_rng(17)
    Hq, Hkv, d, bs = 8, 2, 8, 4
    q, k, v, tables, lens, logical = _paged_case(rng, S=2, Hq=Hq, Hkv=Hkv, d=d, bs=bs, lens=(6, 9))
    G = Hq // Hkv
    k2, v2 = pool.new_pools(k.shape[0], Hq, d, bs, np.float32)
    for s, L in enumerate(lens):
        kt, vt = logical[s]
        rep_k = np.stack([kt[:, h // G] for h in range(Hq)], axis=1).astype(np.float32)
        rep_v = np.stack([vt[:, h // G] for h in range(Hq)], axis=1).astype(np.float32)
        pool.append(k2, v2, rep_k, rep_v, [int(tables[s, t // bs]) * bs + t % bs for t in range(L)])
    a = att.decode_attention(q, k, v, tables, lens)
    b = att.decode_attention(q, k2, v2, tables, lens)
    return np.allclose(a, b, rtol=1e-13, atol=1e-13)


def pin_block_permutation_invariance():
    rng = np.random.default_rng(18)
    q, k, v, tables, lens, logical = _paged_case(rng, S=3, lens=(5, 12, 16))
    bs = k.shape[3]
    k2, v2 = pool.new_pools(k.shape[0], k.shape[1], q.shape[2], bs, np.float32)
    ident = np.full_like(tables, -1)
    nxt = 0
    for s, L in enumerate(lens):  # contiguous placement: identity-like table
        nblk = -(-L // bs)
        ident[s, :nblk] = np.arange(nxt, nxt + nblk)
        nxt += nblk
        kt, vt = logical[s]
        pool.append(k2, v2, kt.astype(np.float32), vt.astype(np.float32),
                    [int(ident[s, t // bs]) * bs + t % bs for t in range(L)])
    a = att.decode_attention(q, k, v, tables, lens)
    b = att.decode_attention(q, k2, v2, ident, lens)
    return np.array_equal(a, b)


def pin_shared_equals_private():
    rng = np.random.default_rng(19)
    d, bs, Hkv, Hq = 8, 4, 1, 2
    k, v = pool.new_pools(12, Hkv, d, bs, np.float32)
    L = 10
    kt = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vt = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    shared = np.array([[0, 1, 2], [0, 1, 2]])
    private = np.array([[0, 1, 2], [3, 4, 5]])
    for row in (0, 1):
        pool.append(k, v, kt, vt, [int(private[row, t // bs]) * bs + t % bs for t in range(L)])
    q = rng.standard_normal((2, Hq, d)).astype(np.float32)
    lens = np.array([L, L])
    return np.array_equal(att.decode_attention(q, k, v, shared, lens), att.decode_attention(q, k, v, private, lens))


def pin_split_merge_equals_unsplit():
    rng = np.random.default_rng(20)
    L, Hq, Hkv, d = 53, 4, 2, 8
    kt = rng.standard_normal((L, Hkv, d))
    vt = rng.standard_normal((L, Hkv, d))
    q = rng.standard_normal((Hq, d))
    full = att.dense_attention(q, kt, vt, 0.3)
    ok = True
    for P in (4, 16, 50, 53, 64):
        m, l, acc = att.partition_partials(q, kt, vt, 0.3, P)
        ok &= np.allclose(att.lse_merge(m, l, acc), full, rtol=1e-12, atol=1e-13)
    # an empty trailing partition must weigh nothing
    m, l, acc = att.partition_partials(q, kt, vt, 0.3, 16)
    m = np.concatenate([m, np.full((1, Hq), -np.inf)])
    l = np.concatenate([l, np.zeros((1, Hq))])
    acc = np.concatenate([acc, np.zeros((1, Hq, d))])
    ok &= np.allclose(att.lse_merge(m, l, acc), full, rtol=1e-12, atol=1e-13)
    return bool(ok)


def pin_zero_length_gives_zero_row():
    rng = np.random.default_rng(21)
    q, k, v, tables, lens, _ = _paged_case(rng, S=2, lens=(3, 6))
    lens = np.array([0, 6])
    out = att.decode_attention(q, k, v, tables, lens)
    return np.array_equal(out[0], np.zeros_like(out[0])) and np.isfinite(out).all()


PINS = [
    pin_bruteforce,
    pin_single_token_returns_v0,
    pin_zero_query_gives_mean,
    pin_equal_keys_give_mean,
    pin_constant_values,
    pin_two_tokens_logistic,
    pin_needle,
    pin_gqa_equals_replicated_mha,
    pin_block_permutation_invariance,
    pin_shared_equals_private,
    pin_split_merge_equals_unsplit,
    pin_zero_length_gives_zero_row,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin()


# ------------------------------------------------------- planted mistakes
def _mut_no_scale(q_row, k_seq, v_seq, scale):
    return _ORIG_DENSE(q_row, k_seq, v_seq, 1.0)


def _mut_gqa_modulo(q_row, k_seq, v_seq, scale):
    Hq, d = q_row.shape
    Hkv = k_seq.shape[1]
    out = np.zeros((Hq, d))
    if k_seq.shape[0] == 0:
        return out
    for h in range(Hq):
        g = h % Hkv
        x = (k_seq[:, g] @ q_row[h]) * scale
        p = np.exp(x - x.max())
        out[h] = (p @ v_seq[:, g]) / p.sum()
    return out


def _mut_k_for_v(q_row, k_seq, v_seq, scale):
    return _ORIG_DENSE(q_row, k_seq, k_seq, scale)


def _mut_no_normalise(q_row, k_seq, v_seq, scale):
    Hq, d = q_row.shape
    G = Hq // k_seq.shape[1]
    out = np.zeros((Hq, d))
    if k_seq.shape[0] == 0:
        return out
    for h in range(Hq):
        x = (k_seq[:, h // G] @ q_row[h]) * scale
        out[h] = np.exp(x - x.max()) @ v_seq[:, h // G]
    return out


def _mut_drop_last_token(q_row, k_seq, v_seq, scale):
    return _ORIG_DENSE(q_row, k_seq[:-1], v_seq[:-1], scale)


def _mut_negated_logits(q_row, k_seq, v_seq, scale):
    return _ORIG_DENSE(q_row, k_seq, v_seq, -scale)


def _mut_gather_slot_order(k_pool, v_pool, table_row, length):
    # reads the slots of each block in reverse order
    kg, vg = _ORIG_GATHER(k_pool, v_pool, table_row, -(-length // k_pool.shape[3]) * k_pool.shape[3])
    bs = k_pool.shape[3]
    kg = kg.reshape(-1, bs, *kg.shape[1:])[:, ::-1].reshape(kg.shape)
    vg = vg.reshape(-1, bs, *vg.shape[1:])[:, ::-1].reshape(vg.shape)
    return kg[:length], vg[:length]


_ORIG_DENSE = att.dense_attention
_ORIG_GATHER = pool.gather

MUTANTS = {
    "no_scale": ("dense", _mut_no_scale),
    "gqa_modulo": ("dense", _mut_gqa_modulo),
    "k_for_v": ("dense", _mut_k_for_v),
    "no_normalise": ("dense", _mut_no_normalise),
    "drop_last_token": ("dense", _mut_drop_last_token),
    "negated_logits": ("dense", _mut_negated_logits),
    "gather_slot_order": ("gather", _mut_gather_slot_order),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    where, fn = MUTANTS[name]
    if where == "dense":
        monkeypatch.setattr(att, "dense_attention", fn)
    else:
        monkeypatch.setattr(pool, "gather", fn)
    failed = []
    for pin in PINS:
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
