"""Pins of the oracle runner's logical K/V view (CPU only).

``OracleRun`` keeps, for every sequence, the source (value key, row) of each
logical token, independently of the pools, and rebuilds a sequence's
contiguous K/V from those sources (``logical_kv``).  That rebuild is the
reference of the full-size GPU checks, where no CPU pool is materialised, so
it must agree with the other way of reading a sequence: gathering its blocks
through its block table from the pools the same script filled.  The pages
state that the engine consults the table to collect the blocks and the
sequence then looks contiguous ("PagedAttention et RadixAttention : parlons
de KV Cache", *PagedAttention : la mémoire comme un système
d'exploitation*, second step).

Every scaled workload script below (plain batches, fork with copy-on-write,
ten growing steps at block size 32, cached admissions of two tenants,
chunked prefill, a swap round trip, radix-indexed conversation turns) is
checked after its setup and after every step: the rebuilt K/V equal the
gathered K/V bit for bit, and the attention computed from either is the
same.  Planted mistakes in the runner's bookkeeping of sources must fail the
pin.
"""
import numpy as np
import pytest

import oracle.attention as oatt
import oracle.pool as opool
from oracle.block_manager import BlockManagerModel
from oracle.radix import RadixCacheModel
from oracle.runner import OracleRun, _storage
from workloads import Workload


def _gathered(run, sid):
    """fp64 K, V of one sequence gathered through its table from the run's pools."""
    n = len(run.bm.tables[sid])
    rows, lens = run.bm.block_tables([sid], max(n, 1))
    L = int(lens[0])
    k, v = opool.gather(run.k_pool, run.v_pool, np.asarray(rows[0]), L)
    return L, opool.to_f64(k), opool.to_f64(v)


def check_logical(run, sids=None):
    """The runner's logical K/V of every sequence equals the pool gather."""
    sids = run.w.decode_seqs if sids is None else sids
    for sid in sids:
        L, kg, vg = _gathered(run, sid)
        assert L == len(run.sources[sid]), f"seq {sid}: {len(run.sources[sid])} sources for length {L}"
        kl, vl = run.logical_kv(sid)
        if L == 0:
            assert kl is None and vl is None
            continue
        assert kl.shape == kg.shape and vl.shape == vg.shape
        assert np.array_equal(kl, kg), f"seq {sid}: logical K differs from the pool gather"
        assert np.array_equal(vl, vg), f"seq {sid}: logical V differs from the pool gather"


def check_attention(run, q):
    """logical_attention of every decode sequence equals attention over the pools."""
    ref = run.attention(q)
    for i in range(run.w.num_seqs):
        got = run.logical_attention(q, i)
        np.testing.assert_allclose(got, ref[i], rtol=1e-12, atol=1e-15, err_msg=f"sequence {i}")


SCALED = {
    "c1": ("c1_tiny_f32", {}),
    "c2": ("c2_8b_bf16", dict(lengths=[300, 17, 1, 64, 129], num_blocks=120)),
    "c3": ("c3_70b_32k_bf16", dict(lengths=[300, 17, 1, 513], num_blocks=130)),
    "c4": ("c4_prefix_bf16", dict(prefix_len=40, num_prompts=3, n_samples=4, suffix_max=30, num_blocks=200)),
    "c5": ("c5_mixed_bs32_bf16", dict(lengths=[16, 40, 33, 100, 1000, 64, 65, 31, 2], num_blocks=80)),
    "c6": ("c6_prefix_cache_bf16", dict(prefix_len=64, num_prompts=6, suffix_max=40, num_blocks=300)),
}


@pytest.mark.parametrize("key", list(SCALED))
def test_logical_kv_equals_pool_gather_every_step(key):
    name, over = SCALED[key]
    w = Workload(name, variant="q64" if name != "c1_tiny_f32" else "plain", overrides=over)
    run = OracleRun(w)
    check_logical(run)
    steps = w.config.steps if key == "c5" else 3
    for k in range(steps):
        run.step(k)
        check_logical(run)
        check_attention(run, w.q(k))
    if key == "c4":
        assert sum(len(p) for p in run.cow_log) > 0, "the script must exercise copy-on-write"
    if key == "c6":
        assert any(n > 0 for n in run.admitted.values()), "the script must find cached prefixes"


def test_logical_prefill_rows_equal_pool_prefill():
    w = Workload("c7_prefill_bf16", variant="q64",
                 overrides=dict(histories=[0, 5, 33, 100], chunks=[1, 17, 40, 64], num_blocks=100))
    run = OracleRun(w)
    check_logical(run)
    for k in range(2):
        run.prefill_step(k)
        check_logical(run)
        q = w.prefill_q(k)
        ref = run.prefill_attention(q)
        for row in range(q.shape[0]):
            np.testing.assert_allclose(run.logical_prefill_row(q, row), ref[row], rtol=1e-12, atol=1e-15,
                                       err_msg=f"chunk {k} row {row}")


def test_logical_kv_survives_swap_round_trip():
    """Swap two sequences out to a host pool, let a new sequence overwrite the
    freed device blocks, swap them back in: their logical K/V (which a swap
    does not change) still equal the gather from the device pool."""
    w = Workload("c2_8b_bf16", variant="q64", overrides=dict(lengths=[300, 77, 1000, 16], num_blocks=160))
    c = w.config
    run = OracleRun(w)
    NH = 100
    run.bm.add_host_pool(NH)
    hk, hv = opool.new_pools(NH, c.num_kv_heads, c.head_dim, c.block_size, np.uint16)
    for sid in (2, 0):
        opool.swap_copy(run.k_pool, run.v_pool, hk, hv, run.bm.swap_out(sid))
    # a new sequence takes the freed blocks and fills them with other rows
    run._apply(("add", 99))
    run._apply(("append", [99], [900], ("prefill", 2)))
    check_logical(run, [1, 3, 99])
    for sid in (0, 2):
        opool.swap_copy(hk, hv, run.k_pool, run.v_pool, run.bm.swap_in(sid))
    check_logical(run, [0, 1, 2, 3, 99])
    run.step(0)
    check_logical(run)
    check_attention(run, w.q(0))


def test_radix_turns_gather_the_conversation():
    """Multi-turn conversations admitted through the radix index (token-granular
    reuse, copy-on-write of a partial block): gathering each turn's sequence
    through its table returns the conversation's own rows, the reference of
    the GPU radix test."""
    w = Workload("c9_multiturn_bf16", overrides=dict(num_convs=3, num_turns=3, user_max=60, resp_max=40,
                                                     num_blocks=200))
    c = w.config
    bm = BlockManagerModel(w.num_blocks, c.block_size, w.free_order)
    rm = RadixCacheModel(bm)
    kp, vp = opool.new_pools(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, np.uint16)
    kv = [w.kv(("conv", i)) for i in range(w.num_convs)]
    toks = [w.conv_tokens(i) for i in range(w.num_convs)]
    copies = 0
    for t in range(w.num_turns):
        sids = [100 * (t + 1) + i for i in range(w.num_convs)]
        for i, sid in enumerate(sids):
            pe, te = w.prompt_end[i][t], w.turn_end[i][t]
            m = rm.admit(sid, toks[i][:pe].tolist())
            k, v = kv[i]
            slots, pairs = bm.append_slots([sid], [te - m])
            copies += len(pairs)
            opool.copy_blocks(kp, vp, pairs)
            opool.append(kp, vp, _storage(k[m:te]), _storage(v[m:te]), slots)
        for i, sid in enumerate(sids):
            te = w.turn_end[i][t]
            rows, lens = bm.block_tables([sid], len(bm.tables[sid]))
            kg, vg = opool.gather(kp, vp, np.asarray(rows[0]), int(lens[0]))
            k, v = kv[i]
            assert int(lens[0]) == te
            assert np.array_equal(kg, _storage(k[:te])) and np.array_equal(vg, _storage(v[:te])), \
                f"turn {t} conversation {i}"
        for i, sid in enumerate(sids):
            rm.insert(sid, toks[i][:w.turn_end[i][t]].tolist())
            rm.release(sid)
            bm.free_seq(sid)
    assert copies > 0


# ---------------------------------------------------------------- planted mistakes
class _ForkShortRun(OracleRun):
    """Mistake: a forked child records one source fewer than it shares."""

    def _apply(self, op):
        if op[0] == "fork":
            _, parent, child, n = op
            self.bm.fork(parent, child, n)
            self.sources[child] = list(self.sources[parent][: n - 1])
            return
        super()._apply(op)


class _ForkShiftedRun(OracleRun):
    """Mistake: a forked child records the parent's sources shifted by one."""

    def _apply(self, op):
        if op[0] == "fork":
            _, parent, child, n = op
            self.bm.fork(parent, child, n)
            src = self.sources[parent]
            self.sources[child] = list(src[1:n]) + [src[n - 1]]
            return
        super()._apply(op)


class _AdmitFromOneRun(OracleRun):
    """Mistake: cached prompt positions recorded as prompt rows 1..n."""

    def _apply(self, op):
        if op[0] == "admit":
            _, sid, tokens, key, salt = op
            tokens = [int(t) for t in tokens]
            n = self.bm.add_seq_cached(sid, tokens, salt)
            self.admitted[sid] = n
            self.sources[sid] = [(key, i + 1) for i in range(n)]
            self._append([sid], [len(tokens) - n], key, token_ids=tokens[n:], first_row=n)
            return
        super()._apply(op)


class _AppendSameRowsRun(OracleRun):
    """Mistake: every sequence of a batched append records the same rows."""

    def _append(self, sids, ntoks, key, token_ids=None, first_row=0):
        slots, pairs = self.bm.append_slots(sids, ntoks, token_ids=token_ids)
        self.cow_log.append(pairs)
        for sid, n in zip(sids, ntoks):
            self.sources[sid].extend((key, first_row + i) for i in range(n))
        opool.copy_blocks(self.k_pool, self.v_pool, pairs)
        k, v = self._kv(key)
        end = first_row + len(slots)
        opool.append(self.k_pool, self.v_pool, _storage(k[first_row:end]), _storage(v[first_row:end]), slots)
        return slots, pairs


@pytest.mark.parametrize("cls,key", [(_ForkShortRun, "c4"), (_ForkShiftedRun, "c4"), (_AdmitFromOneRun, "c6"),
                                     (_AppendSameRowsRun, "c5")])
def test_pin_catches_planted_mistakes(cls, key):
    name, over = SCALED[key]
    w = Workload(name, variant="q64", overrides=over)
    with pytest.raises(AssertionError):
        run = cls(w)
        check_logical(run)
        for k in range(2):
            run.step(k)
            check_logical(run)
