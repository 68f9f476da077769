"""Device-side range checks and the device status word.

Kernels never access memory outside their buffers whatever the device-side
indices hold; an index out of range is skipped (writes) or clamped (decode
reads) and sets a PKV_DEV_* flag that pkv_device_status returns.  In
particular the decode step's append writes nothing for a context length
above max_context_len: a clamped length would name the slot of a token
already in the cache, which may sit in a block other sequences share
("PagedAttention et RadixAttention : parlons de KV Cache", *PagedAttention :
la mémoire comme un système d'exploitation*, fourth step: a shared block is
only ever copied, never written in place).  Both ways the decode call takes
are covered: the append folded into the decode kernel (few sequences) and
the append launched first (more sequences than decode workgroups per kv
head)."""
import numpy as np
import pytest
import torch

from helpers import say

pytestmark = pytest.mark.gpu


def _setup(S, L, bs=16, Hq=8, Hkv=2, d=128, seed=3):
    import paged_kv_cache_230_amd as pkv

    g = torch.Generator().manual_seed(seed)
    nb_seq = -(-L // bs)
    nb = S * nb_seq + 4
    perm = torch.randperm(nb, generator=g)
    tables = perm[: S * nb_seq].view(S, nb_seq).to(torch.int32).cuda()
    k, v = pkv.new_pools(nb, Hkv, d, bs, torch.bfloat16)
    k.copy_((torch.randn(k.shape, generator=g) * 0.1).to(torch.bfloat16))
    v.copy_((torch.randn(v.shape, generator=g) * 0.1).to(torch.bfloat16))
    q = (torch.randn(S, Hq, d, generator=g) * 0.5).to(torch.bfloat16).cuda()
    kn = torch.full((S, Hkv, d), 3.0, dtype=torch.bfloat16, device="cuda")
    return tables, k, v, q, kn


@pytest.mark.parametrize("S", [3, 4000], ids=["folded", "launched"])
def test_append_skips_lengths_above_max_context_len(S):
    """max_context_len one short of the true length: the call reads the
    clamped context, writes no row, and reports the bad length."""
    import paged_kv_cache_230_amd as pkv

    L, bs = 40, 16
    say(f"case device status: append with max_context_len {L - 1} < L = {L}, {S} sequences")
    tables, k, v, q, kn = _setup(S, L)
    wph = pkv.paged_attention_workgroups_per_head(S, 2, 128, bs, L - 1)
    assert (S <= wph) == (S == 3), "the two cases must take the two branches"
    pkv.device_status()  # clear
    k0, v0 = k.clone(), v.clone()
    lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_decode_append(out, q, kn, kn, k, v, tables, lens, L - 1)
    flags = pkv.device_status()
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), k0.view(torch.int16)), "K pool written"
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16)), "V pool written"
    assert flags & pkv.api.N.PKV_DEV_BAD_LENGTH, f"flags {flags}"
    # the output is the decode of the clamped context (L - 1 tokens)
    ref = torch.empty_like(q)
    pkv.paged_attention_decode(ref, q, k, v, tables, torch.full((S,), L - 1, dtype=torch.int32, device="cuda"),
                               L - 1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert pkv.device_status() == 0, "the valid call must leave the word clear"


def test_in_range_calls_leave_the_word_clear():
    import paged_kv_cache_230_amd as pkv

    tables, k, v, q, kn = _setup(5, 100)
    pkv.device_status()
    lens = torch.tensor([100, 1, 0, 37, 64], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_decode_append(out, q, kn, kn, k, v, tables, lens, 100, partition_size=32)
    pkv.paged_kv_append(kn, kn, k, v, torch.tensor([5, -1, 7, 9, 11], dtype=torch.int32, device="cuda"))
    pkv.paged_kv_copy_blocks(k, v, torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"))
    assert pkv.device_status() == 0


def test_out_of_range_indices_are_skipped_and_reported():
    import paged_kv_cache_230_amd as pkv
    N = pkv.api.N

    tables, k, v, q, kn = _setup(3, 40)
    nb = k.shape[0]
    pkv.device_status()
    k0, v0 = k.clone(), v.clone()
    # append: a slot past the pool is skipped
    pkv.paged_kv_append(kn, kn, k, v, torch.tensor([nb * 16, -1, nb * 16 + 5], dtype=torch.int32, device="cuda"))
    assert pkv.device_status() == N.PKV_DEV_BAD_SLOT
    # copy: a pair naming a block past the pool is skipped
    pkv.paged_kv_copy_blocks(k, v, torch.tensor([[0, nb], [nb + 3, 1]], dtype=torch.int32, device="cuda"))
    assert pkv.device_status() == N.PKV_DEV_BAD_PAIR
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), k0.view(torch.int16)) and torch.equal(v.view(torch.int16),
                                                                                   v0.view(torch.int16))
    # decode: a table entry outside the pool is read as block 0 and reported
    bad = tables.clone()
    bad[1, 1] = nb + 100
    lens = torch.full((3,), 40, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_decode(out, q, k, v, bad, lens, 40)
    assert pkv.device_status() == N.PKV_DEV_BAD_BLOCK_ID
    # decode + append: the append's own block out of range writes nothing
    bad = tables.clone()
    bad[2, 2] = -7  # holds position 39, the appended row
    pkv.paged_attention_decode_append(out, q, kn, kn, k, v, bad, lens, 40)
    assert pkv.device_status() & N.PKV_DEV_BAD_BLOCK_ID
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16)[tables[2, 2].item()], k0.view(torch.int16)[tables[2, 2].item()])
    # a negative length
    pkv.paged_attention_decode(out, q, k, v, tables, torch.tensor([40, -3, 40], dtype=torch.int32, device="cuda"),
                               40)
    assert pkv.device_status() == N.PKV_DEV_BAD_LENGTH
    torch.cuda.synchronize()
    assert torch.equal(out[1].float().cpu(), torch.zeros_like(out[1].float().cpu())), "clamped to an empty row"
    # reading without clearing keeps the flags
    pkv.paged_kv_append(kn, kn, k, v, torch.tensor([nb * 16, -1, -1], dtype=torch.int32, device="cuda"))
    assert pkv.device_status(clear=False) == N.PKV_DEV_BAD_SLOT
    assert pkv.device_status() == N.PKV_DEV_BAD_SLOT
    assert pkv.device_status() == 0
