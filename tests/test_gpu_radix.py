"""Radix-tree prefix reuse end to end on the GPU: multi-turn conversations
whose every prompt repeats the conversation so far.  Each turn admits the
prompt through the radix index (token-granular: a match may end inside a
block, whose first write is then copied), appends the rest of the prompt
and the response, decodes all conversations, and inserts the turn for
reuse.  Admissions, slots, copy pairs and pools equal the oracle's bit for
bit; decode outputs equal the oracle over its pool and over each
conversation's logical (contiguous) K/V."""
import numpy as np
import pytest
import torch

from helpers import assert_close, say, storage_np
import oracle.attention as oatt
import oracle.pool as opool
from oracle.block_manager import BlockManagerModel
from oracle.radix import RadixCacheModel
from workloads import Workload

pytestmark = pytest.mark.gpu


def _st(t):
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


def test_multiturn_radix_reuse_and_decode():
    import paged_kv_cache_230_amd as pkv

    w = Workload("c9_multiturn_bf16", variant="q64")
    c = w.config
    cache = pkv.PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, "cuda",
                             w.free_order)
    rx = pkv.RadixIndex(cache.bm)
    bm = BlockManagerModel(w.num_blocks, c.block_size, w.free_order)
    rm = RadixCacheModel(bm)
    ok, ov = opool.new_pools(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, np.uint16)
    kv = [w.kv(("conv", i)) for i in range(w.num_convs)]
    toks = [w.conv_tokens(i) for i in range(w.num_convs)]
    reused = prompt_total = n_copies = 0
    for t in range(w.num_turns):
        sids = [100 * (t + 1) + i for i in range(w.num_convs)]
        for i, sid in enumerate(sids):
            pe, te = w.prompt_end[i][t], w.turn_end[i][t]
            m = rx.admit(sid, toks[i][:pe])
            assert m == rm.admit(sid, toks[i][:pe].tolist())
            if t:
                assert m == w.turn_end[i][t - 1]  # the whole previous conversation, to the token
            reused += m
            prompt_total += pe
            k, v = kv[i]
            slots, pairs = cache.append([sid], [te - m], k[m:te], v[m:te])
            o_slots, o_pairs = bm.append_slots([sid], [te - m])
            assert slots.tolist() == o_slots and pairs.tolist() == [list(p) for p in o_pairs]
            n_copies += len(o_pairs)
            opool.copy_blocks(ok, ov, o_pairs)
            opool.append(ok, ov, _st(k[m:te]), _st(v[m:te]), o_slots)
        q = w.turn_q(t)
        out = cache.decode(q.cuda(), sids)
        torch.cuda.synchronize()
        rows, lens = bm.block_tables(sids, max(len(bm.tables[s]) for s in sids))
        assert_close(out, oatt.decode_attention(_st(q), ok, ov, np.array(rows), np.array(lens)), "bf16",
                     f"turn {t} vs oracle pool")
        for i in range(w.num_convs):
            te = w.turn_end[i][t]
            k, v = kv[i]
            ref = oatt.dense_attention(opool.to_f64(_st(q[i])), opool.to_f64(_st(k[:te])), opool.to_f64(_st(v[:te])),
                                       c.head_dim ** -0.5)
            assert_close(out[i:i + 1], ref[None], "bf16", f"turn {t} conversation {i} vs logical K/V")
        for i, sid in enumerate(sids):
            te = w.turn_end[i][t]
            assert rx.insert(sid, toks[i][:te]) == rm.insert(sid, toks[i][:te].tolist())
            rx.release(sid)
            rm.release(sid)
            cache.bm.free_seq(sid)
            bm.free_seq(sid)
        rm.check_invariants()
    assert np.array_equal(storage_np(cache.k_cache).view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(storage_np(cache.v_cache).view(np.uint8), ov.view(np.uint8))
    assert n_copies > 0  # matches ending inside a block were copied on their first write
    say(f"  reused {reused} of {prompt_total} prompt tokens; {n_copies} partial blocks copied on write")
    rx.close()
