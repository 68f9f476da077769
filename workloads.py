"""Seeded synthetic decode workloads for the paged KV-cache hot path.

This module only *describes* inputs: shapes, context lengths, the initial
order of the free-block pool, a script of sequence operations, and the
random K/V/q values that feed them.  It holds none of the method's
arithmetic (no slot computation, no gathering, no attention): both the
HIP path (through the C-ABI library) and the CPU oracle consume the same
script and the same value bits, and each side executes the script with
its own code.

Values are drawn from torch's CPU generator, one generator per value key
(seeded from the workload seed and the key), so any single sequence's
tokens can be regenerated on its own without drawing the others.

The five workloads follow the configurations the task is measured on:

* ``c1_tiny_f32``  -- 4 sequences, lengths {17, 33, 64, 100}, 4 q / 4 kv
  heads, head_dim 64, block 16, 64 blocks, fp32 N(0, 1).
* ``c2_8b_bf16``   -- Llama-3-8B-shaped layer: 64 sequences, lengths
  uniform in [128, 4096], 32 q / 8 kv heads, head_dim 128, block 16,
  20k-block pool, bf16 N(0, 1)/sqrt(128).
* ``c3_70b_32k_bf16`` -- Llama-3-70B-shaped layer: 16 sequences of 32768
  tokens, 64 q / 8 kv heads, head_dim 128, block 16, 40k-block pool.
* ``c4_prefix_bf16`` -- 50 prompts sharing one 2048-token prefix plus
  private suffixes uniform in [1, 512]; 8 samples forked per prompt, each
  appending one token (copy-on-write of the shared partial block).
* ``c5_mixed_bs32_bf16`` -- 256 sequences, lengths log-uniform in
  [16, 16384], 64 q / 8 kv heads, block 32, pool sized to 95 % occupancy,
  10 consecutive append+decode steps.
* ``c6_prefix_cache_bf16`` -- prefix caching: 50 requests whose prompts
  are one common 2048-token system prompt plus a private user part of
  uniform [1, 512] tokens (token ids uniform in [0, 32000)), spread over 2
  tenants with their own salts; 2 earlier requests (one per tenant) are
  admitted and released first, so the 50 find the system prompt's blocks
  on the eviction list.  8B-shaped heads, block 16, 20k-block pool.
* ``c7_prefill_bf16`` -- chunked prefill: 16 sequences of the 70B-shaped
  layer, each with a cached history of uniform [0, 8192] tokens; every
  step appends a chunk of uniform [128, 1024] new tokens per sequence (the
  same length each step) and runs causal attention of the chunk over the
  whole cache.  Block 16, 48k-block pool.
* ``c8_swap_bf16`` -- swapping: 4 sequences of 32768 tokens of the
  70B-shaped layer (block 16, 10k-block pool) and a host pool holding all
  of them; a step swaps the 4 out to host memory and back in.
* ``c9_multiturn_bf16`` -- multi-turn conversations: 8 conversations of 3
  turns; a turn adds a user message of uniform [20, 400] tokens and a
  response of uniform [10, 200] tokens (ids uniform in [0, 32000)), and a
  turn's prompt is the whole conversation so far plus the new message.
  K/V rows are a function of (conversation, position).  8B-shaped heads,
  block 16, 4k-block pool.

Reading of the length convention: a stated context length is the number of
tokens the decode attention reads *including* the token appended in that
step, so the cache holds ``L - 1`` tokens before the first step.

Script operations (tuples):

* ``("add", sid)``                  -- register an empty sequence
* ``("append", sids, ntoks, key)``  -- append ``ntoks[i]`` tokens to
  ``sids[i]``; K/V come from ``kv(key)`` in sequence-major order
* ``("fork", parent, child, n)``    -- child shares parent's first n tokens
* ``("free", sid)``                 -- release a sequence
* ``("admit", sid, tokens, key, salt)`` -- cached admission of a prompt:
  register ``sid`` sharing the prompt's cached leading blocks, then append
  the rest of the prompt with its token ids; K/V of prompt position ``i``
  are row ``i`` of ``kv(key)``

After the setup script, each of ``steps`` decode steps appends one token to
every sequence of ``decode_seqs`` (values ``kv(("step", k))``) and then
runs decode attention with queries ``q(k)``; ``step_tokens(k)`` gives the
new tokens' ids where the workload tracks them (else None).  A prefill
workload's step instead appends ``chunk_lens[i]`` tokens to each sequence
(values ``kv(("chunk", k))``, sequence-major) and runs causal attention of
those tokens with queries ``prefill_q(k)`` (rows packed by sequence,
offsets ``query_start()``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Config", "Workload", "CONFIGS", "VARIANTS"]


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str  # "f32" or "bf16": storage type of q, K, V and the output
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    value_std: float
    seed: int
    steps: int = 1

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "c1_tiny_f32": Config("c1_tiny_f32", "f32", 4, 4, 64, 16, 1.0, 231),
    "c2_8b_bf16": Config("c2_8b_bf16", "bf16", 32, 8, 128, 16, 128 ** -0.5, 232),
    "c3_70b_32k_bf16": Config("c3_70b_32k_bf16", "bf16", 64, 8, 128, 16, 128 ** -0.5, 233),
    "c4_prefix_bf16": Config("c4_prefix_bf16", "bf16", 32, 8, 128, 16, 128 ** -0.5, 234),
    "c5_mixed_bs32_bf16": Config("c5_mixed_bs32_bf16", "bf16", 64, 8, 128, 32, 128 ** -0.5, 235, steps=10),
    "c6_prefix_cache_bf16": Config("c6_prefix_cache_bf16", "bf16", 32, 8, 128, 16, 128 ** -0.5, 236),
    "c7_prefill_bf16": Config("c7_prefill_bf16", "bf16", 64, 8, 128, 16, 128 ** -0.5, 237),
    "c8_swap_bf16": Config("c8_swap_bf16", "bf16", 64, 8, 128, 16, 128 ** -0.5, 238),
    "c9_multiturn_bf16": Config("c9_multiturn_bf16", "bf16", 32, 8, 128, 16, 128 ** -0.5, 239),
}

# Stress variants of the value distribution (same shapes).  With the
# N(0,1)/sqrt(128) bf16 values the logits have a standard deviation of
# about 0.008, so softmax is nearly uniform; these variants make the score
# path matter: larger query scales, a planted "needle" key, and logits in
# the hundreds (overflow / rescale path).
VARIANTS = ("plain", "q64", "q512", "needle", "large")

_KEY_TAGS = {"prefill": 1, "step": 2, "q": 3, "prefix": 4, "suffix": 5, "needle": 6, "system": 7, "user": 8,
             "system_tokens": 9, "user_tokens": 10, "step_tokens": 11, "chunk": 12, "chunk_q": 13, "conv": 14,
             "conv_tokens": 15, "turn_q": 16}
VOCAB = 32000


def _key_seed(seed: int, key: tuple) -> int:
    tag = _KEY_TAGS[key[0]]
    ints = [seed, tag] + [int(k) for k in key[1:]]
    state = np.random.SeedSequence(ints).generate_state(2, dtype=np.uint32)
    return int(state[0]) | (int(state[1] & 0x7FFFFFFF) << 32)


@dataclass
class Workload:
    """A concrete, seeded instance of one configuration.

    ``overrides`` scales a configuration down for tests (``num_seqs``,
    ``lengths``, ``num_blocks``, ``steps``, ``prefix_len``, ``num_prompts``,
    ``n_samples``, ``suffix_max``); the defaults give the full sizes.
    """

    name: str
    variant: str = "plain"
    seed: int | None = None
    overrides: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.variant not in VARIANTS:
            raise ValueError(f"unknown variant {self.variant!r}")
        base = CONFIGS[self.name]
        if self.seed is not None:
            base = replace(base, seed=self.seed)
        if "steps" in self.overrides:
            base = replace(base, steps=int(self.overrides["steps"]))
        for k in ("num_q_heads", "num_kv_heads", "head_dim", "block_size"):
            if k in self.overrides:
                base = replace(base, **{k: int(self.overrides[k])})
        self.config = base
        rng = np.random.default_rng(base.seed)
        builder = {
            "c1_tiny_f32": self._build_plain_c1,
            "c2_8b_bf16": self._build_plain_c2,
            "c3_70b_32k_bf16": self._build_plain_c3,
            "c4_prefix_bf16": self._build_prefix,
            "c5_mixed_bs32_bf16": self._build_plain_c5,
            "c6_prefix_cache_bf16": self._build_cached,
            "c7_prefill_bf16": self._build_prefill,
            "c8_swap_bf16": self._build_swap,
            "c9_multiturn_bf16": self._build_multiturn,
        }[self.name]
        builder(rng)

    # ------------------------------------------------------------------ build
    def _lengths_override(self, lengths):
        if "lengths" in self.overrides:
            lengths = np.asarray(self.overrides["lengths"], dtype=np.int64)
        elif "num_seqs" in self.overrides:
            lengths = lengths[: int(self.overrides["num_seqs"])]
        return lengths

    def _finish_plain(self, rng, lengths, num_blocks):
        lengths = self._lengths_override(lengths)
        num_blocks = int(self.overrides.get("num_blocks", num_blocks))
        self.num_blocks = num_blocks
        self.free_order = rng.permutation(num_blocks).astype(np.int32)
        self.lengths = lengths.astype(np.int64)
        self.decode_seqs = list(range(len(lengths)))
        ops = [("add", s) for s in self.decode_seqs]
        for s, L in enumerate(lengths):
            if L - 1 > 0:
                ops.append(("append", [s], [int(L - 1)], ("prefill", s)))
        self.setup_ops = ops
        self.prefill_rows = {s: int(L - 1) for s, L in enumerate(lengths)}

    def _build_plain_c1(self, rng):
        self._finish_plain(rng, np.array([17, 33, 64, 100]), 64)

    def _build_plain_c2(self, rng):
        lengths = rng.integers(128, 4096 + 1, size=64)
        self._finish_plain(rng, lengths, 20000)

    def _build_plain_c3(self, rng):
        self._finish_plain(rng, np.full(16, 32768), 40000)

    def _build_plain_c5(self, rng):
        u = rng.uniform(math.log(16), math.log(16384), size=256)
        lengths = np.clip(np.rint(np.exp(u)), 16, 16384).astype(np.int64)
        lengths = self._lengths_override(lengths)
        bs = self.config.block_size
        used = int(sum((int(L) - 1 + bs - 1) // bs for L in lengths))
        num_blocks = int(math.ceil(used / 0.95))
        self._finish_plain(rng, lengths, num_blocks)

    def _build_prefix(self, rng):
        """Shared system prompt + private suffixes, then n samples per prompt.

        Sequence ids: 0 holds the shared prefix; 1..P are the prompts; the
        decode sequences are P+1 .. P + P*n.  Prompts and the prefix holder
        are released once forked, so the prefix blocks end up referenced by
        the samples only.
        """
        o = self.overrides
        prefix_len = int(o.get("prefix_len", 2048))
        num_prompts = int(o.get("num_prompts", 50))
        n_samples = int(o.get("n_samples", 8))
        suffix_max = int(o.get("suffix_max", 512))
        self.prefix_len = prefix_len
        self.suffix_lens = rng.integers(1, suffix_max + 1, size=num_prompts).astype(np.int64)
        self.num_blocks = int(o.get("num_blocks", 20000))
        self.free_order = rng.permutation(self.num_blocks).astype(np.int32)
        ops = [("add", 0), ("append", [0], [prefix_len], ("prefix",))]
        decode = []
        nxt = 1 + num_prompts
        for p in range(num_prompts):
            pid = 1 + p
            ops.append(("fork", 0, pid, prefix_len))
            ops.append(("append", [pid], [int(self.suffix_lens[p])], ("suffix", p)))
            n = prefix_len + int(self.suffix_lens[p])
            for _ in range(n_samples):
                ops.append(("fork", pid, nxt, n))
                decode.append(nxt)
                nxt += 1
            ops.append(("free", pid))
        ops.append(("free", 0))
        self.setup_ops = ops
        self.decode_seqs = decode
        self.lengths = np.array(
            [prefix_len + int(self.suffix_lens[p]) + 1 for p in range(num_prompts) for _ in range(n_samples)],
            dtype=np.int64,
        )

    def _build_cached(self, rng):
        """Cached admissions: warm-up requests admitted and released, then
        the decode requests.  Request r belongs to tenant r % n_tenants."""
        o = self.overrides
        self.prefix_len = int(o.get("prefix_len", 2048))
        n_tenants = int(o.get("n_tenants", 2))
        warm = int(o.get("warm", n_tenants))
        num_prompts = int(o.get("num_prompts", 50))
        suffix_max = int(o.get("suffix_max", 512))
        self.n_tenants = n_tenants
        self.salts = [int(x) for x in rng.integers(1, 2 ** 62, size=n_tenants)]
        n_req = warm + num_prompts
        self.suffix_lens = rng.integers(1, suffix_max + 1, size=n_req).astype(np.int64)
        self.num_blocks = int(o.get("num_blocks", 20000))
        self.free_order = rng.permutation(self.num_blocks).astype(np.int32)
        admit = lambda r: ("admit", r, self.prompt_tokens(r), ("prompt", r), self.salts[r % n_tenants])
        ops = [admit(r) for r in range(warm)]
        ops += [("free", r) for r in range(warm)]
        ops += [admit(r) for r in range(warm, n_req)]
        self.setup_ops = ops
        self.decode_seqs = list(range(warm, n_req))
        self.lengths = np.array([self.prefix_len + int(self.suffix_lens[r]) + 1 for r in self.decode_seqs],
                                dtype=np.int64)
        self.tracks_tokens = True

    def _build_multiturn(self, rng):
        """Turn t of conversation c: prompt = positions [0, prompt_end[c][t]),
        then the response up to turn_end[c][t]."""
        o = self.overrides
        n_conv = int(o.get("num_convs", 8))
        n_turns = int(o.get("num_turns", 3))
        users = rng.integers(int(o.get("user_min", 20)), int(o.get("user_max", 400)) + 1, size=(n_conv, n_turns))
        resps = rng.integers(int(o.get("resp_min", 10)), int(o.get("resp_max", 200)) + 1, size=(n_conv, n_turns))
        self.num_blocks = int(o.get("num_blocks", 4000))
        self.free_order = rng.permutation(self.num_blocks).astype(np.int32)
        self.num_convs, self.num_turns = n_conv, n_turns
        self.prompt_end, self.turn_end = [], []
        for c in range(n_conv):
            pe, te, end = [], [], 0
            for t in range(n_turns):
                end += int(users[c, t])
                pe.append(end)
                end += int(resps[c, t])
                te.append(end)
            self.prompt_end.append(pe)
            self.turn_end.append(te)
        self.conv_len = [te[-1] for te in self.turn_end]
        self.setup_ops = []
        self.decode_seqs = list(range(n_conv))
        self.lengths = np.array(self.conv_len, dtype=np.int64)

    def conv_tokens(self, c: int) -> np.ndarray:
        """Token ids of conversation c, every position of every turn."""
        return self._ints(("conv_tokens", c), self.conv_len[c])

    def turn_q(self, t: int):
        """Queries of the last token of turn t, one row per conversation."""
        cfg = self.config
        shape = (self.num_convs, cfg.num_q_heads, cfg.head_dim)
        return self._randn(("turn_q", t), shape, cfg.value_std * self._q_scale()).to(cfg.torch_dtype)

    def _build_swap(self, rng):
        lengths = np.full(int(self.overrides.get("num_seqs", 4)), 32768)
        self._finish_plain(rng, lengths, 10000)
        self.host_blocks = int(self.overrides.get("host_blocks", len(lengths) * 2048 + 64))

    def _build_prefill(self, rng):
        """Histories in the cache, then chunks of new tokens every step."""
        o = self.overrides
        S = int(o.get("num_seqs", 16))
        hist = rng.integers(0, int(o.get("history_max", 8192)) + 1, size=S).astype(np.int64)
        chunks = rng.integers(int(o.get("chunk_min", 128)), int(o.get("chunk_max", 1024)) + 1, size=S)
        if "histories" in o:
            hist = np.asarray(o["histories"], dtype=np.int64)
        if "chunks" in o:
            chunks = np.asarray(o["chunks"], dtype=np.int64)
        self.num_blocks = int(o.get("num_blocks", 48000))
        self.free_order = rng.permutation(self.num_blocks).astype(np.int32)
        self.chunk_lens = [int(c) for c in chunks]
        self.decode_seqs = list(range(len(hist)))
        ops = [("add", s) for s in self.decode_seqs]
        for s, h in enumerate(hist):
            if h > 0:
                ops.append(("append", [s], [int(h)], ("prefill", s)))
        self.setup_ops = ops
        self.prefill_rows = {s: int(h) for s, h in enumerate(hist)}
        self.lengths = (hist + chunks).astype(np.int64)  # context of the first step's chunks

    def query_start(self):
        """Row offsets of the sequences' chunks in ``prefill_q`` (int64 ``[S+1]``)."""
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int64)

    def prefill_q(self, step: int):
        """Queries of step ``step``'s chunks ``[sum(chunk_lens)][num_q_heads][head_dim]``."""
        c = self.config
        shape = (int(sum(self.chunk_lens)), c.num_q_heads, c.head_dim)
        return self._randn(("chunk_q", step), shape, c.value_std * self._q_scale()).to(c.torch_dtype)

    def _ints(self, key, n):
        g = torch.Generator().manual_seed(_key_seed(self.config.seed, key))
        return torch.randint(0, VOCAB, (n,), generator=g, dtype=torch.int64).numpy()

    def prompt_tokens(self, r: int) -> np.ndarray:
        """Token ids of request r's prompt: the system prompt, then its own part."""
        return np.concatenate([self._ints(("system_tokens",), self.prefix_len),
                               self._ints(("user_tokens", r), int(self.suffix_lens[r]))])

    def step_tokens(self, k: int):
        """Ids of the tokens decode step k appends (one per decode sequence), or None."""
        if not getattr(self, "tracks_tokens", False):
            return None
        return self._ints(("step_tokens", k), self.num_seqs)

    # ----------------------------------------------------------------- values
    @property
    def num_seqs(self) -> int:
        return len(self.decode_seqs)

    def _randn(self, key, shape, std):
        g = torch.Generator().manual_seed(_key_seed(self.config.seed, key))
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        return x

    def _k_scale(self) -> float:
        # "large": keys x32 with queries x512 give logits with a standard
        # deviation near 130; values keep the configuration's distribution.
        return 32.0 if self.variant == "large" else 1.0

    def _q_scale(self) -> float:
        return {"plain": 1.0, "q64": 64.0, "q512": 512.0, "needle": 1.0, "large": 512.0}[self.variant]

    def kv(self, key: tuple):
        """K and V rows ``[T][num_kv_heads][head_dim]`` for one script key."""
        c = self.config
        if key[0] == "prefill":
            T = self.prefill_rows[int(key[1])]
        elif key[0] == "prefix":
            T = self.prefix_len
        elif key[0] == "suffix":
            T = int(self.suffix_lens[int(key[1])])
        elif key[0] == "step":
            T = self.num_seqs
        elif key[0] == "prompt":
            # the system prompt's rows are the same for every request
            ks, vs = self.kv(("system",))
            ku, vu = self.kv(("user", int(key[1])))
            return torch.cat([ks, ku]), torch.cat([vs, vu])
        elif key[0] == "chunk":
            T = int(sum(self.chunk_lens))
        elif key[0] == "conv":
            T = self.conv_len[int(key[1])]
        elif key[0] == "system":
            T = self.prefix_len
        elif key[0] == "user":
            T = int(self.suffix_lens[int(key[1])])
        else:
            raise KeyError(key)
        shape = (T, c.num_kv_heads, c.head_dim)
        k = self._randn(key + (0,), shape, c.value_std * self._k_scale())
        v = self._randn(key + (1,), shape, c.value_std)
        if self.variant == "needle" and key[0] == "prefill" and T > 0:
            # Plant, in every kv head, a key equal to 8x the first query head
            # of its group (step-0 query) at one seeded position.
            s = int(key[1])
            pos = self.needle_position(s)
            q0 = self.q(0)[self.decode_seqs.index(s)].to(torch.float32)
            G = c.num_q_heads // c.num_kv_heads
            for g in range(c.num_kv_heads):
                k[pos, g] = 8.0 * q0[g * G]
        return k.to(c.torch_dtype), v.to(c.torch_dtype)

    def needle_position(self, s: int) -> int:
        g = torch.Generator().manual_seed(_key_seed(self.config.seed, ("needle", s)))
        T = self.prefill_rows[s]
        return int(torch.randint(0, T, (1,), generator=g).item())

    def q(self, step: int):
        """Queries ``[num_seqs][num_q_heads][head_dim]`` for decode step ``step``."""
        c = self.config
        shape = (self.num_seqs, c.num_q_heads, c.head_dim)
        x = self._randn(("q", step), shape, c.value_std * self._q_scale())
        return x.to(c.torch_dtype)

    def token_count(self) -> int:
        """Rows appended by the setup script (for sizing)."""
        n = 0
        for op in self.setup_ops:
            if op[0] == "append":
                n += sum(op[2])
            elif op[0] == "admit":
                n += len(op[2])
        return n
