"""Seeded synthetic inputs for the paged decode path.

This module is the one place both sides of a parity check get their inputs
from.  It draws context lengths, a physical block permutation, block tables
and N(0,1) query/key/value values; it performs no attention, softmax, slot or
cache arithmetic, and hands out no slot: where a test needs slots, the
library side takes them from its allocator and the oracle side from its own
walk of the tables.  The one place it reads the tables is ``filled_mask``,
which decides which pool slots get values and which NaN; a mistake there
would put NaN where a token should be, and every parity test requires finite
outputs.  Everything is a function of ``seed``: integer structure
(lengths, permutation, tables, tails, allocator start order) comes from
``numpy.random.default_rng(seed)``, floating-point values from a
``torch.Generator`` seeded with the same number on the requested device, drawn
as float32 and rounded to the KV dtype (round-to-nearest-even).

The pages measured on ShareGPT request lengths and LLaMA weights, neither of
which is available; the length laws below stand in for them (uniform for the
tiny and long-context cases, lognormal around the stated median for the
LLaMA-shaped ones), and q/K/V are standard normal.

Pool content convention ("pre-step" pool): a sequence of context length ``ctx``
has its first ``ctx - 1`` tokens already in the pool; the slot of token
``ctx - 1`` (the one the decode step writes), the unfilled tail of every last
block and every block no sequence owns hold NaN, so that any read of them
shows up in the output.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

KV_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# Named workloads.  Shapes follow the LLaMA-7B / 13B / 70B attention layers the
# pages' evaluation is quoted on (page "PagedAttention: the KV cache was the
# bottleneck all along", section "The number that made us read the code").
CONFIGS = {
    "tiny": dict(S=4, Hq=4, Hkv=4, D=64, dtype="f32", bs=16, NB=64,
                 lengths=("uniform", 1, 100), partition_tokens=0),
    # Partitioning is a launch choice, not part of the workload's arithmetic:
    # the 7B batch has 2048 (sequence, head) pairs with lognormal lengths, and
    # splitting contexts into 512-token pieces evens out the workgroups.
    "llama7b": dict(S=64, Hq=32, Hkv=32, D=128, dtype="f16", bs=16, NB=16384,
                    lengths=("lognormal", 500, 0.5, 16, 2048), partition_tokens=512),
    # NB is chosen per block size so that the pool holds 262144 tokens.
    "llama13b": dict(S=128, Hq=40, Hkv=40, D=128, dtype="bf16", bs=16, NB=None,
                     pool_tokens=262144, lengths=("lognormal", 700, 0.5, 1, 2048),
                     partition_tokens=0),
    "long_gqa": dict(S=8, Hq=64, Hkv=8, D=128, dtype="bf16", bs=16, NB=16384,
                     lengths=("uniform", 16384, 32768), partition_tokens=512),
}

SHARED_PREFIX = dict(prompts=16, samples=4, Hq=40, Hkv=40, D=128, dtype="f16", bs=16,
                     NB=4096, prompt_len=512, tail=(0, 256))


def draw_lengths(rng: np.random.Generator, law, S: int) -> np.ndarray:
    """Context lengths (tokens attended, the step's new token included)."""
    kind = law[0]
    if kind == "uniform":
        lo, hi = law[1], law[2]
        x = rng.integers(lo, hi + 1, size=S)
    elif kind == "lognormal":
        median, sigma, lo, hi = law[1:]
        x = np.rint(np.exp(rng.normal(np.log(median), sigma, size=S)))
        x = np.clip(x, lo, hi)
    elif kind == "fixed":                 # one value for all, or one per sequence
        x = np.broadcast_to(np.asarray(law[1], dtype=np.int64), (S,)).copy()
    else:
        raise ValueError(f"unknown length law {law!r}")
    return x.astype(np.int32)


def _randn(shape, gen, device, dtype_name: str) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).to(
        KV_DTYPES[dtype_name])


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclasses.dataclass
class DecodeWorkload:
    """One decode step over a batch of sequences whose K/V live in a paged pool."""
    name: str
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    dtype: str
    scale: float                 # float32 value handed to both sides
    partition_tokens: int
    context_lens: np.ndarray     # int32 [S]
    block_tables: np.ndarray     # int32 [S, MB], -1 past the sequence's blocks
    block_order: np.ndarray      # int32 [NB] the permutation the tables were cut from
    q: torch.Tensor              # [S, Hq, D]
    key_cache: torch.Tensor      # [NB, Hkv, bs, D] pre-step
    value_cache: torch.Tensor    # [NB, Hkv, bs, D] pre-step
    new_key: torch.Tensor        # [S, Hkv, D]  token ctx-1 of each sequence
    new_value: torch.Tensor      # [S, Hkv, D]

    @property
    def MB(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def paged_tables(rng: np.random.Generator, lens: np.ndarray, bs: int, NB: int,
                 MB: Optional[int] = None):
    """Assign each sequence ceil(ctx/bs) physical blocks, consecutively from one
    random permutation of the pool (so neighbours in a table are scattered).
    Returns (tables, permutation)."""
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    if int(nblk.sum()) > NB:
        raise ValueError(f"pool of {NB} blocks cannot hold {int(nblk.sum())}")
    perm = rng.permutation(NB).astype(np.int32)
    mb = int(nblk.max()) if MB is None else int(MB)
    tables = np.full((len(lens), max(mb, 1)), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += n
    return tables, perm


def filled_mask(tables: np.ndarray, filled: np.ndarray, bs: int, NB: int) -> np.ndarray:
    """bool [NB, bs]: True where a slot holds one of the first ``filled[s]`` tokens."""
    mask = np.zeros((NB, bs), dtype=bool)
    for s in range(tables.shape[0]):
        n = int(filled[s])
        j = 0
        while n > 0:
            mask[tables[s, j], :min(n, bs)] = True
            n -= bs
            j += 1
    return mask


def make_decode(name: str, seed: int = 0, device="cpu", **over) -> DecodeWorkload:
    """Build a named decode workload; keyword overrides replace config fields
    (e.g. ``S=6`` for a reduced-size parity case, ``bs=8`` for the sweep)."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    S, Hq, Hkv, D, bs = cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["bs"]
    NB = cfg["NB"] if cfg.get("NB") else cfg["pool_tokens"] // bs
    rng = np.random.default_rng(seed)
    lens = draw_lengths(rng, cfg["lengths"], S)
    tables, perm = paged_tables(rng, lens, bs, NB, cfg.get("MB"))
    mask = filled_mask(tables, np.maximum(lens.astype(np.int64) - 1, 0), bs, NB)
    gen = _generator(seed, device)
    dt = cfg["dtype"]
    q = _randn((S, Hq, D), gen, device, dt)
    pools = []
    poison = ~torch.from_numpy(mask).to(device)[:, None, :, None]
    for _ in range(2):
        p = torch.randn(NB, Hkv, bs, D, generator=gen, device=device, dtype=torch.float32)
        p.masked_fill_(poison, float("nan"))
        pools.append(p.to(KV_DTYPES[dt]))
        del p
    nk = _randn((S, Hkv, D), gen, device, dt)
    nv = _randn((S, Hkv, D), gen, device, dt)
    return DecodeWorkload(
        name=name, seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, dtype=dt,
        scale=float(np.float32(1.0 / np.sqrt(D))),
        partition_tokens=int(cfg.get("partition_tokens", 0)),
        context_lens=lens, block_tables=tables, block_order=perm, q=q,
        key_cache=pools[0], value_cache=pools[1], new_key=nk, new_value=nv)


@dataclasses.dataclass
class SharedPrefixScript:
    """Parallel sampling over shared prompts: each prompt is prefilled into its
    own sequence, forked into ``samples`` sequences, and every sample then
    grows by its own tail before one final decode step over all samples."""
    seed: int
    prompts: int
    samples: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    dtype: str
    scale: float
    prompt_len: int
    tails: np.ndarray            # int32 [prompts*samples] tokens appended after the fork
    init_order: np.ndarray       # int32 [NB] order in which free blocks are handed out
    prompt_k: torch.Tensor       # [prompts, prompt_len, Hkv, D]
    prompt_v: torch.Tensor
    tail_k: torch.Tensor         # [S, max_tail, Hkv, D]
    tail_v: torch.Tensor
    step_k: torch.Tensor         # [S, Hkv, D]  final step's token
    step_v: torch.Tensor
    q: torch.Tensor              # [S, Hq, D]
    key_cache: torch.Tensor      # [NB, Hkv, bs, D] initial pool, all NaN
    value_cache: torch.Tensor

    @property
    def S(self) -> int:
        return self.prompts * self.samples

    def seq_id(self, prompt: int, sample: int) -> int:
        return prompt * self.samples + sample


def make_shared_prefix(seed: int = 0, device="cpu", **over) -> SharedPrefixScript:
    cfg = dict(SHARED_PREFIX)
    cfg.update(over)
    rng = np.random.default_rng(seed)
    P, M = cfg["prompts"], cfg["samples"]
    S = P * M
    lo, hi = cfg["tail"]
    tails = rng.integers(lo, hi + 1, size=S).astype(np.int32)
    NB = cfg["NB"]
    init_order = rng.permutation(NB).astype(np.int32)
    gen = _generator(seed, device)
    dt, Hkv, Hq, D, L = cfg["dtype"], cfg["Hkv"], cfg["Hq"], cfg["D"], cfg["prompt_len"]
    mt = int(tails.max()) if S else 0
    pk = _randn((P, L, Hkv, D), gen, device, dt)
    pv = _randn((P, L, Hkv, D), gen, device, dt)
    tk = _randn((S, mt, Hkv, D), gen, device, dt)
    tv = _randn((S, mt, Hkv, D), gen, device, dt)
    sk = _randn((S, Hkv, D), gen, device, dt)
    sv = _randn((S, Hkv, D), gen, device, dt)
    q = _randn((S, Hq, D), gen, device, dt)
    kc = torch.full((NB, Hkv, cfg["bs"], D), float("nan"), device=device,
                    dtype=KV_DTYPES[dt])
    vc = kc.clone()
    return SharedPrefixScript(
        seed=seed, prompts=P, samples=M, Hq=Hq, Hkv=Hkv, D=D, bs=cfg["bs"], NB=NB,
        dtype=dt, scale=float(np.float32(1.0 / np.sqrt(D))), prompt_len=L, tails=tails,
        init_order=init_order, prompt_k=pk, prompt_v=pv, tail_k=tk, tail_v=tv,
        step_k=sk, step_v=sv, q=q, key_cache=kc, value_cache=vc)


# Forked batches (parallel sampling and beam search, page "PagedAttention: the
# KV cache was the bottleneck all along", section "Virtual memory for
# attention"): every sample of a prompt holds the prompt's full blocks in its
# table; pairs of samples share a few more whole blocks (a later fork at a
# block boundary, as beams do); the rest of each context is private.
# Unforked sequences are mixed in, and the batch order is shuffled.
FORKED = dict(prompts=4, samples=4, singles=3, Hq=32, Hkv=4, D=128, dtype="bf16", bs=16,
              prompt_len=(100, 700), tail=(0, 300), pair_blocks=(0, 3), single_len=(1, 900),
              slack_blocks=8)


def make_forked(seed: int = 0, device="cpu", **over) -> DecodeWorkload:
    """A decode workload whose block tables share physical blocks the way
    forked sequences do; pool content as for :func:`make_decode`."""
    cfg = dict(FORKED)
    cfg.update(over)
    rng = np.random.default_rng(seed)
    bs, P, M = cfg["bs"], cfg["prompts"], cfg["samples"]
    rows, lens = [], []
    next_id = [0]

    def fresh(n):
        ids = list(range(next_id[0], next_id[0] + n))
        next_id[0] += n
        return ids

    for _ in range(P):
        plen = int(rng.integers(cfg["prompt_len"][0], cfg["prompt_len"][1] + 1))
        prompt = fresh(plen // bs)
        pair = []
        for j in range(M):
            if j % 2 == 0:
                pair = fresh(int(rng.integers(cfg["pair_blocks"][0], cfg["pair_blocks"][1] + 1)))
            shared = prompt + pair
            ctx = plen + int(rng.integers(cfg["tail"][0], cfg["tail"][1] + 1)) + 1
            ctx = max(ctx, len(shared) * bs + 1)          # shared blocks lie before ctx-1
            rows.append(shared + fresh(-(-ctx // bs) - len(shared)))
            lens.append(ctx)
    for _ in range(cfg["singles"]):
        ctx = int(rng.integers(cfg["single_len"][0], cfg["single_len"][1] + 1))
        rows.append(fresh(-(-ctx // bs)))
        lens.append(ctx)
    S = len(rows)
    order = rng.permutation(S)
    NB = next_id[0] + cfg["slack_blocks"]
    perm = rng.permutation(NB).astype(np.int32)            # logical id -> physical block
    MB = max(len(r) for r in rows)
    tables = np.full((S, MB), -1, dtype=np.int32)
    ctx_lens = np.zeros(S, dtype=np.int32)
    for dst, src in enumerate(order):
        tables[dst, :len(rows[src])] = perm[rows[src]]
        ctx_lens[dst] = lens[src]
    mask = filled_mask(tables, np.maximum(ctx_lens.astype(np.int64) - 1, 0), bs, NB)
    gen = _generator(seed, device)
    dt, Hq, Hkv, D = cfg["dtype"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    q = _randn((S, Hq, D), gen, device, dt)
    pools = []
    poison = ~torch.from_numpy(mask).to(device)[:, None, :, None]
    for _ in range(2):
        p = torch.randn(NB, Hkv, bs, D, generator=gen, device=device, dtype=torch.float32)
        p.masked_fill_(poison, float("nan"))
        pools.append(p.to(KV_DTYPES[dt]))
    nk = _randn((S, Hkv, D), gen, device, dt)
    nv = _randn((S, Hkv, D), gen, device, dt)
    return DecodeWorkload(
        name="forked", seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, dtype=dt,
        scale=float(np.float32(1.0 / np.sqrt(D))), partition_tokens=0,
        context_lens=ctx_lens, block_tables=tables, block_order=perm, q=q,
        key_cache=pools[0], value_cache=pools[1], new_key=nk, new_value=nv)


# Requests that share a system prompt (page "PagedAttention: the KV cache was
# the bottleneck all along", section "What is left": common system prompts
# across users; page "Efficient Memory Management for Large Language Model
# Serving with PagedAttention", from the abstract: sharing across requests).
# Every request's prompt is the same system prompt followed by its own text.
SYSTEM_PROMPT = dict(requests=64, Hq=40, Hkv=40, D=128, dtype="bf16", bs=16, NB=8192,
                     system_len=1024, own=(16, 512))


@dataclasses.dataclass
class SystemPromptScript:
    seed: int
    requests: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    dtype: str
    scale: float
    system_len: int
    own_lens: np.ndarray          # int32 [R] tokens after the system prompt
    init_order: np.ndarray        # int32 [NB]
    system_k: torch.Tensor        # [system_len, Hkv, D]
    system_v: torch.Tensor
    own_k: torch.Tensor           # [R, max_own, Hkv, D]
    own_v: torch.Tensor
    step_k: torch.Tensor          # [R, Hkv, D] the decode step's token
    step_v: torch.Tensor
    q: torch.Tensor               # [R, Hq, D]
    key_cache: torch.Tensor       # [NB, Hkv, bs, D] initial pool, all NaN
    value_cache: torch.Tensor

    def system_keys(self) -> list:
        """One registry key per full block of the system prompt (standing in
        for a hash chained over its token ids)."""
        return [(1 << 40) + j for j in range(self.system_len // self.bs)]

    def prompt(self, r: int):
        """Request r's whole prompt, K and V [system_len + own, Hkv, D]."""
        n = int(self.own_lens[r])
        return (torch.cat([self.system_k, self.own_k[r, :n]]),
                torch.cat([self.system_v, self.own_v[r, :n]]))


def make_system_prompt(seed: int = 0, device="cpu", **over) -> SystemPromptScript:
    cfg = dict(SYSTEM_PROMPT)
    cfg.update(over)
    rng = np.random.default_rng(seed)
    R, bs, NB = cfg["requests"], cfg["bs"], cfg["NB"]
    own = rng.integers(cfg["own"][0], cfg["own"][1] + 1, size=R).astype(np.int32)
    init_order = rng.permutation(NB).astype(np.int32)
    gen = _generator(seed, device)
    dt, Hkv, Hq, D, L = cfg["dtype"], cfg["Hkv"], cfg["Hq"], cfg["D"], cfg["system_len"]
    mo = int(own.max()) if R else 0
    sk = _randn((L, Hkv, D), gen, device, dt)
    sv = _randn((L, Hkv, D), gen, device, dt)
    ok = _randn((R, mo, Hkv, D), gen, device, dt)
    ov = _randn((R, mo, Hkv, D), gen, device, dt)
    tk = _randn((R, Hkv, D), gen, device, dt)
    tv = _randn((R, Hkv, D), gen, device, dt)
    q = _randn((R, Hq, D), gen, device, dt)
    kc = torch.full((NB, Hkv, bs, D), float("nan"), device=device, dtype=KV_DTYPES[dt])
    return SystemPromptScript(
        seed=seed, requests=R, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, dtype=dt,
        scale=float(np.float32(1.0 / np.sqrt(D))), system_len=L, own_lens=own,
        init_order=init_order, system_k=sk, system_v=sv, own_k=ok, own_v=ov, step_k=tk,
        step_v=tv, q=q, key_cache=kc, value_cache=kc.clone())


# Beam search (page "PagedAttention: the KV cache was the bottleneck all
# along", section "Virtual memory for attention": beams share more than
# parallel samples and are forked and discarded all the time).  There are no
# model scores, so which beams survive is drawn at random: at every step each
# of a request's W new beams picks its parent uniformly among the W current
# ones (with replacement), so some beams fork and others are dropped.
BEAM = dict(requests=3, width=4, layers=3, Hq=8, Hkv=4, D=128, dtype="bf16", bs=8, NB=1024,
            prompt=(40, 90), steps=12)


@dataclasses.dataclass
class BeamScript:
    seed: int
    requests: int
    width: int
    layers: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    dtype: str
    scale: float
    steps: int
    prompt_lens: np.ndarray       # int32 [R]
    choices: np.ndarray           # int32 [steps, R, W] parent index of each new beam
    init_order: np.ndarray        # int32 [NB]
    prompt_k: list                # R tensors [layers, prompt_len, Hkv, D]
    prompt_v: list
    step_k: torch.Tensor          # [steps, layers, R*W, Hkv, D] each step's new token
    step_v: torch.Tensor
    q: torch.Tensor               # [layers, R*W, Hq, D] queries of the final step
    key_cache: torch.Tensor       # [NB, Hkv, bs, D] initial pool of every layer, all NaN
    value_cache: torch.Tensor


def make_beam(seed: int = 0, device="cpu", **over) -> BeamScript:
    cfg = dict(BEAM)
    cfg.update(over)
    rng = np.random.default_rng(seed)
    R, W, L, T = cfg["requests"], cfg["width"], cfg["layers"], cfg["steps"]
    lens = rng.integers(cfg["prompt"][0], cfg["prompt"][1] + 1, size=R).astype(np.int32)
    choices = rng.integers(0, W, size=(T, R, W)).astype(np.int32)
    init_order = rng.permutation(cfg["NB"]).astype(np.int32)
    gen = _generator(seed, device)
    dt, Hkv, Hq, D = cfg["dtype"], cfg["Hkv"], cfg["Hq"], cfg["D"]
    pk = [_randn((L, int(n), Hkv, D), gen, device, dt) for n in lens]
    pv = [_randn((L, int(n), Hkv, D), gen, device, dt) for n in lens]
    sk = _randn((T, L, R * W, Hkv, D), gen, device, dt)
    sv = _randn((T, L, R * W, Hkv, D), gen, device, dt)
    q = _randn((L, R * W, Hq, D), gen, device, dt)
    kc = torch.full((cfg["NB"], Hkv, cfg["bs"], D), float("nan"), device=device,
                    dtype=KV_DTYPES[dt])
    return BeamScript(seed=seed, requests=R, width=W, layers=L, Hq=Hq, Hkv=Hkv, D=D,
                      bs=cfg["bs"], NB=cfg["NB"], dtype=dt,
                      scale=float(np.float32(1.0 / np.sqrt(D))), steps=T, prompt_lens=lens,
                      choices=choices, init_order=init_order, prompt_k=pk, prompt_v=pv,
                      step_k=sk, step_v=sv, q=q, key_cache=kc, value_cache=kc.clone())


# Prefill batches: each sequence has ``prefix`` tokens already cached (an
# earlier chunk, or blocks taken from other requests) and a chunk of new
# tokens whose K/V are stored before the attention runs.  The default shape
# is a LLaMA-13B attention layer with lognormal prompt lengths around the
# pages' median, whole prompts (prefix 0).
PREFILL = dict(S=16, Hq=40, Hkv=40, D=128, dtype="bf16", bs=16, NB=None, pool_tokens=65536,
               prefix=("fixed", 0), chunk=("lognormal", 700, 0.5, 16, 2048))


@dataclasses.dataclass
class PrefillWorkload:
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    dtype: str
    scale: float
    chunk_lens: np.ndarray       # int32 [S] new tokens per sequence
    context_lens: np.ndarray     # int32 [S] prefix + chunk
    query_start: np.ndarray      # int32 [S+1] packed row offsets of the chunks
    block_tables: np.ndarray     # int32 [S, MB]
    block_order: np.ndarray      # int32 [NB] the permutation the tables were cut from
    q: torch.Tensor              # [T, Hq, D]
    key_cache: torch.Tensor      # [NB, Hkv, bs, D]: prefixes stored, the rest NaN
    value_cache: torch.Tensor
    new_key: torch.Tensor        # [T, Hkv, D] the chunks' K/V (to be stored)
    new_value: torch.Tensor

    @property
    def T(self) -> int:
        return int(self.query_start[-1])

    @property
    def MB(self) -> int:
        return int(self.block_tables.shape[1])


def make_prefill(seed: int = 0, device="cpu", **over) -> PrefillWorkload:
    cfg = dict(PREFILL)
    cfg.update(over)
    S, Hq, Hkv, D, bs = cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["bs"]
    NB = cfg["NB"] if cfg.get("NB") else cfg["pool_tokens"] // bs
    rng = np.random.default_rng(seed)
    prefix = draw_lengths(rng, cfg["prefix"], S)
    chunk = draw_lengths(rng, cfg["chunk"], S)
    ctx = (prefix + chunk).astype(np.int32)
    tables, perm = paged_tables(rng, ctx, bs, NB, cfg.get("MB"))
    mask = filled_mask(tables, prefix.astype(np.int64), bs, NB)
    gen = _generator(seed, device)
    dt = cfg["dtype"]
    T = int(chunk.sum())
    q = _randn((T, Hq, D), gen, device, dt)
    pools = []
    poison = ~torch.from_numpy(mask).to(device)[:, None, :, None]
    for _ in range(2):
        p = torch.randn(NB, Hkv, bs, D, generator=gen, device=device, dtype=torch.float32)
        p.masked_fill_(poison, float("nan"))
        pools.append(p.to(KV_DTYPES[dt]))
        del p
    nk = _randn((T, Hkv, D), gen, device, dt)
    nv = _randn((T, Hkv, D), gen, device, dt)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    return PrefillWorkload(seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, dtype=dt,
                           scale=float(np.float32(1.0 / np.sqrt(D))), chunk_lens=chunk,
                           context_lens=ctx, query_start=qs, block_tables=tables,
                           block_order=perm, q=q, key_cache=pools[0], value_cache=pools[1],
                           new_key=nk, new_value=nv)


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """Host copy of a KV-dtype tensor as its raw storage: float32 / float16 as
    themselves, bfloat16 as its uint16 bit patterns (numpy has no bfloat16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_numpy_storage(a: np.ndarray, dtype: str, device="cpu") -> torch.Tensor:
    """Inverse of :func:`to_numpy_storage`."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
