"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case draws its inputs from ``paged_kv_cache_198_amd.synth`` (seeded);
the oracle sees the same inputs as host arrays and never anything the HIP
path produced.  Integer work (slots from the allocator, block tables, cache
writes, block copies) must match bit for bit, whole pools included (their
NaN poison too); decode outputs must be within the stated max-abs-error
bound of the float64 oracle: 1e-5 for float32 KV, 2e-3 for float16,
1e-2 for bfloat16 (float32 accumulation, output rounded to the KV dtype).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.alloc as oa
import oracle.decode as od
import paged_kv_cache_198_amd as pa
from paged_kv_cache_198_amd import synth
from prefill_slots import lib_prefill_slots, oracle_prefill_slots

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
DEV = "cuda"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw storage bits, so NaN poison compares equal to itself."""
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


# ---------------------------------------------------------------------------
# one decode step through the library
# ---------------------------------------------------------------------------
def lib_slots(w):
    """Step slots from the C++ allocator: a pool handing out blocks in the
    workload's order, each sequence grown to its context length."""
    alloc = pa.Allocator(w.NB, w.bs, init_order=w.block_order)
    step = np.empty(w.S, dtype=np.int64)
    for s in range(w.S):
        alloc.create(s)
        slots, src, dst = alloc.append_n(s, int(w.context_lens[s]))
        assert (src, dst) == (-1, -1)
        step[s] = slots[-1]
    tables, lens = alloc.build_batch(list(range(w.S)), w.MB)
    return step, tables, lens


def run_step(w, partition_tokens=None, kc=None, vc=None):
    """pa_reshape_and_cache of the step's token, then pa_decode_attention."""
    part = w.partition_tokens if partition_tokens is None else partition_tokens
    step, tables, lens = lib_slots(w)
    assert np.array_equal(tables, w.block_tables)          # allocator reproduces the layout
    assert np.array_equal(lens, w.context_lens)
    kc = w.key_cache.clone() if kc is None else kc
    vc = w.value_cache.clone() if vc is None else vc
    slots_d = torch.from_numpy(step).to(DEV)
    tables_d = torch.from_numpy(tables).to(DEV)
    lens_d = torch.from_numpy(lens).to(DEV)
    out = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
    ws = pa.make_workspace(w.S, w.Hq, w.D, w.max_context_len, part)
    pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc, slots_d)
    pa.pa_decode_attention(out, w.q, kc, vc, tables_d, lens_d, w.max_context_len, w.scale,
                           part, ws)
    torch.cuda.synchronize()
    return out, kc, vc, step


def oracle_step(w, seqs=None, lens=None, write=True):
    """Oracle slots, cache write and fp64 decode on host copies of the inputs
    (sub-pool of the blocks the chosen sequences reference).  ``lens``
    replaces the context lengths; ``write=False`` attends without storing
    the new token."""
    seqs = list(range(w.S)) if seqs is None else list(seqs)
    all_lens = w.context_lens if lens is None else np.asarray(lens)
    need = [-(-int(all_lens[s]) // w.bs) for s in seqs]
    blocks = np.unique(np.concatenate([w.block_tables[s, :n] for s, n in zip(seqs, need)]))
    remap = {int(b): i for i, b in enumerate(blocks)}
    idx = torch.from_numpy(blocks.astype(np.int64)).to(w.key_cache.device)
    kc = synth.to_numpy_storage(w.key_cache.index_select(0, idx))
    vc = synth.to_numpy_storage(w.value_cache.index_select(0, idx))
    tab = np.full((len(seqs), w.MB), -1, dtype=np.int64)
    for i, (s, n) in enumerate(zip(seqs, need)):
        tab[i, :n] = [remap[int(b)] for b in w.block_tables[s, :n]]
    lens = all_lens[seqs]
    sel = torch.tensor(seqs, device=w.new_key.device)
    if write:
        slots = [od.slot_of(tab[i], int(lens[i]) - 1, w.bs) for i in range(len(seqs))]
        kc, vc = od.reshape_and_cache(synth.to_numpy_storage(w.new_key.index_select(0, sel)),
                                      synth.to_numpy_storage(w.new_value.index_select(0, sel)),
                                      kc, vc, slots, inplace=True)
    q = synth.to_numpy_storage(w.q.index_select(0, sel))
    out = od.paged_decode(q, kc, vc, tab, lens, w.scale, w.dtype)
    if not write:
        return out, None
    # the oracle's own slot for every sequence, in full-pool numbering
    full_slots = [od.slot_of(w.block_tables[s], int(lens[i]) - 1, w.bs)
                  for i, s in enumerate(seqs)]
    return out, np.array(full_slots, dtype=np.int64)


def widened(t: torch.Tensor, dtype: str) -> np.ndarray:
    return od.widen(synth.to_numpy_storage(t), dtype)


def check_decode(w, part=None, seqs=None, tol=None):
    note(f"case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} bs={w.bs} NB={w.NB} "
         f"{w.dtype} part={w.partition_tokens if part is None else part} "
         f"max_ctx={w.max_context_len}")
    out, kc, vc, step = run_step(w, part)
    seqs = list(range(w.S)) if seqs is None else list(seqs)
    ref, oslots = oracle_step(w, seqs)
    assert np.array_equal(step[seqs], oslots)                # slots bit-exact
    got = widened(out, w.dtype)[seqs]
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    bound = TOL[w.dtype] if tol is None else tol
    note(f"  max abs err {err:.3e} (bound {bound:g}), max |out| {np.max(np.abs(ref)):.3f}")
    assert err <= bound
    return out, kc, vc, step


# ---------------------------------------------------------------------------
# decode parity on the five workloads (reduced sizes: every output; full
# sizes: every output the oracle can afford, else a sample)
# ---------------------------------------------------------------------------
def test_tiny_full():
    w = synth.make_decode("tiny", device=DEV)
    _, kc, vc, step = check_decode(w)
    # the cache write touched exactly the step slots: compare whole pools
    ref_k, ref_v = od.reshape_and_cache(synth.to_numpy_storage(w.new_key),
                                        synth.to_numpy_storage(w.new_value),
                                        synth.to_numpy_storage(w.key_cache),
                                        synth.to_numpy_storage(w.value_cache), step)
    assert np.array_equal(synth.to_numpy_storage(kc).view(np.uint32), ref_k.view(np.uint32))
    assert np.array_equal(synth.to_numpy_storage(vc).view(np.uint32), ref_v.view(np.uint32))


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_seeds_partitioned(seed):
    w = synth.make_decode("tiny", seed=seed, device=DEV, S=7, NB=96)
    check_decode(w, part=32)
    check_decode(w, part=16)


def test_llama7b_reduced():
    w = synth.make_decode("llama7b", device=DEV, S=8, NB=1024)
    check_decode(w)


def test_llama7b_full():
    w = synth.make_decode("llama7b", device=DEV)
    check_decode(w)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_llama13b_reduced(bs):
    w = synth.make_decode("llama13b", device=DEV, bs=bs, S=6, pool_tokens=16384)
    check_decode(w)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_llama13b_full(bs):
    w = synth.make_decode("llama13b", device=DEV, bs=bs)
    check_decode(w)


@pytest.mark.parametrize("bs", [16, 32])
def test_llama13b_full_partitioned(bs):
    w = synth.make_decode("llama13b", device=DEV, bs=bs)
    check_decode(w, part=256, seqs=range(0, w.S, 3))


def test_long_gqa_reduced():
    w = synth.make_decode("long_gqa", device=DEV, S=3, NB=1024, lengths=("uniform", 700, 4000))
    check_decode(w)                 # 512-token partitions + reduce
    check_decode(w, part=0)         # single pass


def test_long_gqa_full():
    w = synth.make_decode("long_gqa", device=DEV)
    check_decode(w)


@pytest.mark.parametrize("G", [2, 4])
def test_grouped_heads(G):
    w = synth.make_decode("llama7b", device=DEV, S=5, NB=512, Hkv=4, Hq=4 * G,
                          lengths=("uniform", 1, 900))
    check_decode(w)
    check_decode(w, part=128)


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("f16", 64), ("bf16", 64), ("f32", 64)])
def test_dtype_head_dim_grid(dtype, D):
    w = synth.make_decode("llama7b", device=DEV, S=5, NB=512, Hq=4, Hkv=4, D=D, dtype=dtype,
                          lengths=("uniform", 1, 1200))
    check_decode(w)
    check_decode(w, part=256)


@pytest.mark.parametrize("name,over,part", [
    # 16 or more partitions take the wide partition reduce; ragged counts
    # (1, a few, many) in one batch, both head dims, every dtype, both kernels
    ("long_gqa", dict(S=4, NB=2048, lengths=("fixed", [1, 33, 1100, 4000])), 64),
    ("long_gqa", dict(S=3, NB=2048, bs=8, dtype="f16", lengths=("fixed", [4000, 17, 2049])), 32),
    ("llama13b", dict(S=6, bs=16, pool_tokens=16384,
                      lengths=("fixed", [1, 32, 33, 511, 512, 2048])), 32),
    ("llama7b", dict(S=5, NB=512, Hq=4, Hkv=4, D=64, dtype="f32", lengths=("uniform", 1, 900)), 32),
    ("llama7b", dict(S=5, NB=512, Hq=8, Hkv=2, dtype="f16", lengths=("uniform", 300, 1500)), 64),
])
def test_many_partitions(name, over, part):
    w = synth.make_decode(name, device=DEV, **over)
    assert -(-w.max_context_len // part) >= 16
    check_decode(w, part=part)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_length_one_is_exact():
    """Softmax over one token is 1: the output is that token's value row,
    bit for bit (every dtype)."""
    for dt in ("f32", "f16", "bf16"):
        w = synth.make_decode("llama7b", device=DEV, S=9, NB=64, dtype=dt,
                              lengths=("fixed", [1] * 9))
        out, _, _, _ = run_step(w)
        G = w.Hq // w.Hkv
        expect = w.new_value.repeat_interleave(G, dim=1)
        assert torch.equal(bits(out), bits(expect)), dt


def test_block_and_partition_boundaries():
    bs = 16
    lens = [1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1024]
    w = synth.make_decode("llama13b", device=DEV, bs=bs, S=len(lens), pool_tokens=8192,
                          lengths=("fixed", lens))
    for part in (0, 256, 512):
        check_decode(w, part=part)


def test_max_context_fills_table():
    """Contexts that use every table column, MB * bs tokens."""
    w = synth.make_decode("llama13b", device=DEV, bs=8, S=3, pool_tokens=8192,
                          lengths=("fixed", [2048, 2048, 5]))
    assert w.MB * w.bs == 2048
    check_decode(w)
    check_decode(w, part=512)


def test_padding_entries_are_not_read():
    """Table entries past a sequence's blocks may hold anything."""
    w = synth.make_decode("llama7b", device=DEV, S=6, NB=512, lengths=("uniform", 1, 300))
    base, _, _, _ = run_step(w)
    t = w.block_tables.copy()
    t[t < 0] = 2 ** 30                       # far outside the pool
    lens_d = torch.from_numpy(w.context_lens).to(DEV)
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    step, _, _ = lib_slots(w)
    pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc, torch.from_numpy(step).to(DEV))
    out = torch.empty_like(base)
    pa.pa_decode_attention(out, w.q, kc, vc, torch.from_numpy(t).to(DEV), lens_d,
                           w.max_context_len, w.scale, 0, None)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(base))


def test_physical_placement_is_invisible():
    """Relabelling physical blocks changes nothing, bit for bit: the kernel's
    reduction order depends on logical positions only."""
    w = synth.make_decode("llama13b", device=DEV, S=5, pool_tokens=16384,
                          lengths=("uniform", 1, 2000))
    out1, _, _, _ = run_step(w)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(w.NB)).to(DEV)
    inv = torch.argsort(perm)
    w2 = synth.make_decode("llama13b", device=DEV, S=5, pool_tokens=16384,
                           lengths=("uniform", 1, 2000))
    # block b moves to inv[b]
    w2.key_cache = w.key_cache[perm]
    w2.value_cache = w.value_cache[perm]
    inv_np = inv.cpu().numpy()
    w2.block_tables = np.where(w.block_tables >= 0, inv_np[np.maximum(w.block_tables, 0)], -1)
    w2.block_order = inv_np[w.block_order].astype(np.int32)
    out2, _, _, _ = run_step(w2)
    assert torch.equal(bits(out1), bits(out2))


def test_block_size_is_invisible():
    """The same logical tokens at bs 8, 16, 32 give bit-identical outputs
    (contexts under 8192 tokens: no table-chunk boundary inside)."""
    outs = []
    for bs in (8, 16, 32):
        w = synth.make_decode("llama13b", device=DEV, bs=bs, S=4, pool_tokens=16384,
                              lengths=("fixed", [5, 700, 1500, 2048]))
        # rebuild the pools so that every block size holds the same logical values
        rng = torch.Generator(device=DEV).manual_seed(11)
        Kc = torch.randn(4, 2048, w.Hkv, w.D, generator=rng, device=DEV).to(torch.bfloat16)
        Vc = torch.randn(4, 2048, w.Hkv, w.D, generator=rng, device=DEV).to(torch.bfloat16)
        kc = torch.full_like(w.key_cache, float("nan"))
        vc = torch.full_like(w.value_cache, float("nan"))
        for s in range(4):
            n = int(w.context_lens[s]) - 1
            for j in range(-(-n // bs)):
                b = int(w.block_tables[s, j])
                m = min(bs, n - j * bs)
                kc[b, :, :m] = Kc[s, j * bs:j * bs + m].transpose(0, 1)
                vc[b, :, :m] = Vc[s, j * bs:j * bs + m].transpose(0, 1)
        w.key_cache, w.value_cache = kc, vc
        w.q = torch.randn(4, w.Hq, w.D, generator=rng, device=DEV).to(torch.bfloat16)
        w.new_key = Kc[torch.arange(4), torch.tensor(w.context_lens - 1, dtype=torch.long)]
        w.new_value = Vc[torch.arange(4), torch.tensor(w.context_lens - 1, dtype=torch.long)]
        out, _, _, _ = run_step(w)
        outs.append(out)
    assert torch.equal(bits(outs[0]), bits(outs[1])) and torch.equal(bits(outs[0]), bits(outs[2]))


# ---------------------------------------------------------------------------
# cache write and block copy, bit for bit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f16", 64, 8), ("f32", 128, 32)])
def test_cache_write_prefill(dtype, D, bs):
    """Many tokens at once (a prompt), some slots -1, whole pools compared."""
    NB, Hkv, T = 300, 6, 2000
    rng = np.random.default_rng(3)
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.1] = -1
    g = torch.Generator(device=DEV).manual_seed(5)
    kc = torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).to(synth.KV_DTYPES[dtype])
    vc = torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).to(synth.KV_DTYPES[dtype])
    k = torch.randn(T, Hkv, D, generator=g, device=DEV).to(synth.KV_DTYPES[dtype])
    v = torch.randn(T, Hkv, D, generator=g, device=DEV).to(synth.KV_DTYPES[dtype])
    ref_k, ref_v = od.reshape_and_cache(synth.to_numpy_storage(k), synth.to_numpy_storage(v),
                                        synth.to_numpy_storage(kc), synth.to_numpy_storage(vc),
                                        slots)
    pa.pa_reshape_and_cache(k, v, kc, vc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(synth.to_numpy_storage(kc), ref_k)
    assert np.array_equal(synth.to_numpy_storage(vc), ref_v)


def test_cache_write_both_store_policies():
    """The cache write streams its stores out when the rows fit in 32 MiB and
    uses the default policy above that: one call over 34 MB of rows and the
    same rows as two calls of 17 MB leave bit-identical pools, equal to the
    oracle's cache write (some slots -1)."""
    NB, Hkv, bs, D, T = 1200, 40, 16, 128, 1700    # 2 * T * Hkv * D * 2 B = 34.8 MB
    rng = np.random.default_rng(11)
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.05] = -1
    g = torch.Generator(device=DEV).manual_seed(13)
    kc0 = torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).to(torch.bfloat16)
    vc0 = torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(T, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(T, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    s_d = torch.from_numpy(slots).to(DEV)
    kc1, vc1 = kc0.clone(), vc0.clone()
    pa.pa_reshape_and_cache(k, v, kc1, vc1, s_d)                     # one call, default stores
    kc2, vc2 = kc0.clone(), vc0.clone()
    h = T // 2
    pa.pa_reshape_and_cache(k[:h].contiguous(), v[:h].contiguous(), kc2, vc2, s_d[:h].contiguous())
    pa.pa_reshape_and_cache(k[h:].contiguous(), v[h:].contiguous(), kc2, vc2, s_d[h:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(bits(kc1), bits(kc2)) and torch.equal(bits(vc1), bits(vc2))
    ref_k, ref_v = od.reshape_and_cache(synth.to_numpy_storage(k), synth.to_numpy_storage(v),
                                        synth.to_numpy_storage(kc0), synth.to_numpy_storage(vc0),
                                        slots)
    assert np.array_equal(synth.to_numpy_storage(kc1), ref_k)
    assert np.array_equal(synth.to_numpy_storage(vc1), ref_v)


def test_copy_blocks_layers():
    L, NB, Hkv, bs, D = 20, 64, 4, 16, 128        # 20 layers: two launches of layers
    g = torch.Generator(device=DEV).manual_seed(9)
    ks = [torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).half() for _ in range(L)]
    vs = [torch.randn(NB, Hkv, bs, D, generator=g, device=DEV).half() for _ in range(L)]
    rng = np.random.default_rng(4)
    blocks = rng.permutation(NB)
    pairs = np.stack([blocks[:30], blocks[30:60]], axis=1)   # 30 independent pairs
    ref_k, ref_v = od.copy_blocks([synth.to_numpy_storage(t) for t in ks],
                                  [synth.to_numpy_storage(t) for t in vs], pairs)
    pa.pa_copy_blocks(ks, vs, pairs)
    torch.cuda.synchronize()
    for lk, lv, rk, rv in zip(ks, vs, ref_k, ref_v):
        assert np.array_equal(synth.to_numpy_storage(lk), rk)
        assert np.array_equal(synth.to_numpy_storage(lv), rv)


def test_copy_blocks_many_pairs():
    NB, L = 600, 1                                 # 250 pairs: three launches of pairs
    g = torch.Generator(device=DEV).manual_seed(2)
    ks = [torch.randn(NB, 2, 8, 64, generator=g, device=DEV).to(torch.bfloat16)]
    vs = [torch.randn(NB, 2, 8, 64, generator=g, device=DEV).to(torch.bfloat16)]
    blocks = np.random.default_rng(8).permutation(NB)
    pairs = np.stack([blocks[:250], blocks[250:500]], axis=1)
    ref_k, ref_v = od.copy_blocks([synth.to_numpy_storage(ks[0])],
                                  [synth.to_numpy_storage(vs[0])], pairs)
    pa.pa_copy_blocks(ks, vs, pairs)
    torch.cuda.synchronize()
    assert np.array_equal(synth.to_numpy_storage(ks[0]), ref_k[0])
    assert np.array_equal(synth.to_numpy_storage(vs[0]), ref_v[0])


# ---------------------------------------------------------------------------
# shared-prefix parallel sampling: allocator, copy-on-write, cache writes and
# decode, library and oracle each driving their own side
# ---------------------------------------------------------------------------
def drive_shared_prefix_lib(sc):
    kc, vc = sc.key_cache.clone(), sc.value_cache.clone()
    alloc = pa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    log = []
    for i in range(sc.prompts):
        sid = sc.seq_id(i, 0)
        alloc.create(sid)
        slots, _, _ = alloc.append_n(sid, sc.prompt_len)
        pa.pa_reshape_and_cache(sc.prompt_k[i], sc.prompt_v[i], kc, vc,
                                torch.from_numpy(slots).to(DEV))
        for j in range(1, sc.samples):
            alloc.fork(sid, sc.seq_id(i, j))
    steps = int(sc.tails.max()) + 1
    for t in range(steps):
        last = t == steps - 1
        who = [s for s in range(sc.S) if last or t < sc.tails[s]]
        pairs, slots = [], []
        for s in who:
            slot, src, dst = alloc.append(s)
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        log.append((t, slots, pairs))
        if pairs:
            pa.pa_copy_blocks([kc], [vc], pairs)
        sel = torch.tensor(who, device=DEV)
        if last:
            k, v = sc.step_k.index_select(0, sel), sc.step_v.index_select(0, sel)
        else:
            k = sc.tail_k[:, t].index_select(0, sel)
            v = sc.tail_v[:, t].index_select(0, sel)
        pa.pa_reshape_and_cache(k.contiguous(), v.contiguous(), kc, vc,
                                torch.tensor(slots, dtype=torch.int64, device=DEV))
    MB = max(-(-alloc.seq_len(s) // sc.bs) for s in range(sc.S))
    tables, lens = alloc.build_batch(list(range(sc.S)), MB)
    out = torch.empty(sc.S, sc.Hq, sc.D, dtype=sc.q.dtype, device=DEV)
    pa.pa_decode_attention(out, sc.q, kc, vc, torch.from_numpy(tables).to(DEV),
                           torch.from_numpy(lens).to(DEV), int(lens.max()), sc.scale, 0, None)
    torch.cuda.synchronize()
    return out, kc, vc, tables, lens, log, alloc.export()


def drive_shared_prefix_oracle(sc):
    kc = synth.to_numpy_storage(sc.key_cache)
    vc = synth.to_numpy_storage(sc.value_cache)
    pk, pv = synth.to_numpy_storage(sc.prompt_k), synth.to_numpy_storage(sc.prompt_v)
    tk, tv = synth.to_numpy_storage(sc.tail_k), synth.to_numpy_storage(sc.tail_v)
    sk, sv = synth.to_numpy_storage(sc.step_k), synth.to_numpy_storage(sc.step_v)
    alloc = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    log = []
    for i in range(sc.prompts):
        sid = sc.seq_id(i, 0)
        alloc.create(sid)
        slots = [alloc.append(sid)[0] for _ in range(sc.prompt_len)]
        od.reshape_and_cache(pk[i], pv[i], kc, vc, slots, inplace=True)
        for j in range(1, sc.samples):
            alloc.fork(sid, sc.seq_id(i, j))
    steps = int(sc.tails.max()) + 1
    for t in range(steps):
        last = t == steps - 1
        who = [s for s in range(sc.S) if last or t < sc.tails[s]]
        pairs, slots = [], []
        for s in who:
            slot, src, dst = alloc.append(s)
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        log.append((t, slots, pairs))
        od.copy_blocks([kc], [vc], pairs, inplace=True)
        if last:
            k, v = sk[who], sv[who]
        else:
            k, v = tk[who, t], tv[who, t]
        od.reshape_and_cache(k, v, kc, vc, slots, inplace=True)
    MB = max(-(-alloc.seq_len(s) // sc.bs) for s in range(sc.S))
    tables, lens = alloc.build_batch(list(range(sc.S)), MB)
    out = od.paged_decode(synth.to_numpy_storage(sc.q), kc, vc, np.array(tables),
                          np.array(lens), sc.scale, sc.dtype)
    return out, kc, vc, np.array(tables), np.array(lens), log, (list(alloc.ref),
                                                                 alloc.free_stack())


@pytest.mark.parametrize("prompt_len,full", [(504, False), (512, False), (504, True),
                                             (512, True)])
def test_shared_prefix(prompt_len, full):
    kw = {} if full else dict(prompts=3, NB=512, tail=(0, 40))
    sc = synth.make_shared_prefix(device=DEV, prompt_len=prompt_len, **kw)
    note(f"case shared_prefix prompts={sc.prompts} prompt_len={prompt_len} NB={sc.NB} "
         f"tails max {int(sc.tails.max())}")
    out, kc, vc, tables, lens, log, exp = drive_shared_prefix_lib(sc)
    ref, rkc, rvc, rtables, rlens, rlog, rexp = drive_shared_prefix_oracle(sc)
    assert log == rlog                                       # slots and CoW pairs
    assert np.array_equal(tables, rtables) and np.array_equal(lens, rlens)
    assert exp[0] == rexp[0] and exp[1] == rexp[1]           # refcounts, free stack
    # pools, NaN poison included: compare raw bits
    assert np.array_equal(synth.to_numpy_storage(kc).view(np.uint16), rkc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(vc).view(np.uint16), rvc.view(np.uint16))
    copies = sum(len(p) for _, _, p in log)
    expect_copies = 0 if prompt_len % sc.bs == 0 else sum(
        min(int(np.sum((sc.tails[i * sc.samples:(i + 1) * sc.samples] >= 0))), sc.samples - 1)
        for i in range(sc.prompts))
    assert copies == expect_copies
    got = widened(out, sc.dtype)
    err = float(np.max(np.abs(got - ref)))
    note(f"  copies {copies}, max abs err {err:.3e}")
    assert err <= TOL[sc.dtype]


# ---------------------------------------------------------------------------
# grouped heads on the matrix cores (G = 8, D = 128, bf16 / f16): block sizes,
# partitions (every multiple of bs takes the MFMA kernel)
# and lengths around tile, block and partition edges
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,bs,part", [("bf16", 8, 512), ("bf16", 32, 0), ("f16", 16, 512),
                                           ("f16", 16, 0), ("bf16", 16, 96), ("bf16", 16, 48),
                                           ("f16", 8, 64), ("bf16", 8, 24), ("f16", 16, 80),
                                           ("bf16", 32, 96), ("f16", 64, 192), ("bf16", 8, 40)])
def test_gqa_matrix_core(dtype, bs, part):
    # every partition size (a multiple of bs) takes the matrix-core kernel
    w = synth.make_decode("long_gqa", device=DEV, S=4, NB=2048, bs=bs, dtype=dtype,
                          lengths=("uniform", 1, 3000))
    check_decode(w, part=part)


@pytest.mark.parametrize("dtype,D,part", [("f32", 128, 0), ("f32", 128, 48), ("bf16", 64, 96),
                                          ("f16", 64, 0)])
def test_grouped_eight_vector_alu(dtype, D, part):
    # G = 8 outside the matrix-core set (float32, or D = 64) runs on the
    # vector ALUs
    w = synth.make_decode("long_gqa", device=DEV, S=4, NB=2048, dtype=dtype, D=D,
                          lengths=("uniform", 1, 2000))
    check_decode(w, part=part)


def test_gqa_matrix_core_edges():
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1024, 1025]
    w = synth.make_decode("long_gqa", device=DEV, S=len(lens), NB=4096, lengths=("fixed", lens))
    for part in (0, 32, 128, 512):
        check_decode(w, part=part)


def test_gqa_matrix_core_length_one_exact():
    w = synth.make_decode("long_gqa", device=DEV, S=5, NB=64, lengths=("fixed", [1] * 5))
    out, _, _, _ = run_step(w)
    expect = w.new_value.repeat_interleave(w.Hq // w.Hkv, dim=1)
    assert torch.equal(bits(out), bits(expect))


# ---------------------------------------------------------------------------
# fused step: pa_decode_step must equal pa_reshape_and_cache + pa_decode_attention
# bit for bit (outputs and whole pools), on both kernels, with and without
# partitions, and the oracle bound must hold for it directly
# ---------------------------------------------------------------------------
def run_fused(w, part):
    step, tables, lens = lib_slots(w)
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    out = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
    ws = pa.make_workspace(w.S, w.Hq, w.D, w.max_context_len, part)
    pa.pa_decode_step(out, w.q, w.new_key, w.new_value, kc, vc, torch.from_numpy(tables).to(DEV),
                      torch.from_numpy(lens).to(DEV), w.max_context_len, w.scale, part, ws)
    torch.cuda.synchronize()
    return out, kc, vc


FUSED_CASES = [
    ("tiny", {}, 0), ("tiny", dict(S=7, NB=96), 32),
    ("llama13b", dict(bs=8, S=6, pool_tokens=16384), 0),
    ("llama13b", dict(bs=16, S=6, pool_tokens=16384), 256),
    ("llama13b", dict(bs=32, S=6, pool_tokens=16384, lengths=("fixed", [1, 32, 33, 64, 700, 2048])), 0),
    ("llama7b", dict(S=5, NB=512, Hq=4, Hkv=4, D=128, dtype="f32", lengths=("uniform", 1, 900)), 0),
    ("long_gqa", dict(S=3, NB=1024, lengths=("uniform", 700, 4000)), 512),
    ("long_gqa", dict(S=4, NB=1024, lengths=("fixed", [1, 31, 32, 1025])), 0),
    ("long_gqa", dict(S=3, NB=2048, bs=8, dtype="f16", lengths=("uniform", 1, 3000)), 64),
]


@pytest.mark.parametrize("name,over,part", FUSED_CASES)
def test_fused_step_equals_two_calls(name, over, part):
    w = synth.make_decode(name, device=DEV, **over)
    note(f"case fused {name} {over} part={part}")
    out1, kc1, vc1, _ = run_step(w, part)
    out2, kc2, vc2 = run_fused(w, part)
    assert torch.equal(bits(out1), bits(out2))
    assert torch.equal(bits(kc1), bits(kc2)) and torch.equal(bits(vc1), bits(vc2))


def test_fused_step_against_oracle():
    w = synth.make_decode("llama13b", device=DEV, S=8, pool_tokens=16384)
    out, _, _ = run_fused(w, 0)
    ref, _ = oracle_step(w)
    err = float(np.max(np.abs(widened(out, w.dtype) - ref)))
    note(f"  fused max abs err {err:.3e}")
    assert err <= TOL[w.dtype]


CLAMP_CASES = [  # vector-ALU and matrix-core kernels, single pass and partitioned
    ("llama13b", dict(bs=16, S=6, pool_tokens=16384), 0),
    ("llama13b", dict(bs=8, S=6, pool_tokens=16384), 256),
    ("llama7b", dict(S=5, NB=512, Hq=8, Hkv=2, D=64, dtype="f16", lengths=("uniform", 40, 900)), 0),
    ("long_gqa", dict(S=4, NB=1024, lengths=("uniform", 700, 4000)), 512),
    ("long_gqa", dict(S=4, NB=1024, bs=32, dtype="f16", lengths=("uniform", 100, 3000)), 0),
]


@pytest.mark.parametrize("name,over,part", CLAMP_CASES)
def test_fused_step_clamped_lengths(name, over, part):
    """Lengths above max_context_len, and one past the table's reach: the
    fused step stores each new row where a separate cache write would (none
    for the one past the table) and attends the clamped range; outputs and
    whole pools equal the two-call path bit for bit, and the oracle's own
    cache write and decode over the clamped lengths."""
    w = synth.make_decode(name, device=DEV, **over)
    step, tables, lens = lib_slots(w)
    order = np.argsort(w.context_lens)
    big = int(order[-1])                          # its length goes past the table
    # clamps the longer half; the long one's clamped range holds filled rows
    cap = min(int(w.context_lens[order[len(order) // 2]]), int(w.context_lens[big]) - 1)
    lens2 = lens.copy()
    lens2[big] = w.MB * w.bs + 3
    slots = step.copy()
    slots[big] = -1                               # no slot exists past the table
    note(f"case clamp {name} {over} part={part} cap={cap} lens={lens2.tolist()}")
    t_d, l_d = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens2).to(DEV)
    ws = pa.make_workspace(w.S, w.Hq, w.D, cap, part)
    kc1, vc1 = w.key_cache.clone(), w.value_cache.clone()
    out1 = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
    pa.pa_reshape_and_cache(w.new_key, w.new_value, kc1, vc1, torch.from_numpy(slots).to(DEV))
    pa.pa_decode_attention(out1, w.q, kc1, vc1, t_d, l_d, cap, w.scale, part, ws)
    kc2, vc2 = w.key_cache.clone(), w.value_cache.clone()
    out2 = torch.full_like(out1, float("nan"))
    pa.pa_decode_step(out2, w.q, w.new_key, w.new_value, kc2, vc2, t_d, l_d, cap, w.scale,
                      part, ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(out2))
    assert torch.equal(bits(kc1), bits(kc2)) and torch.equal(bits(vc1), bits(vc2))
    # the oracle: slot of position c-1 through the table where it exists,
    # then attention over min(c, cap, MB*bs) tokens
    oslots = [od.slot_of(w.block_tables[s], int(lens2[s]) - 1, w.bs)
              if (int(lens2[s]) - 1) // w.bs < w.MB else -1 for s in range(w.S)]
    assert np.array_equal(np.asarray(oslots, dtype=np.int64), slots)
    okc, ovc = od.reshape_and_cache(synth.to_numpy_storage(w.new_key),
                                    synth.to_numpy_storage(w.new_value),
                                    synth.to_numpy_storage(w.key_cache),
                                    synth.to_numpy_storage(w.value_cache), oslots)
    u8 = lambda a: np.ascontiguousarray(a).view(np.uint8)    # NaN poison compares too
    assert np.array_equal(u8(synth.to_numpy_storage(kc2)), u8(okc))
    assert np.array_equal(u8(synth.to_numpy_storage(vc2)), u8(ovc))
    att = np.minimum(lens2, min(cap, w.MB * w.bs))
    ref = od.paged_decode(synth.to_numpy_storage(w.q), okc, ovc, w.block_tables, att, w.scale,
                          w.dtype)
    got = widened(out2, w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype]


ZERO_CASES = [  # vector-ALU (MHA and grouped) and matrix-core kernels, one pass and split
    ("llama7b", dict(S=6, NB=512, Hq=4, Hkv=4, lengths=("fixed", [0, 17, 0, 300, 1, 0])), 0),
    ("llama7b", dict(S=6, NB=512, Hq=8, Hkv=2, D=64, dtype="bf16",
                     lengths=("fixed", [0, 700, 0, 33, 1, 0])), 64),
    ("long_gqa", dict(S=5, NB=512, lengths=("fixed", [0, 700, 0, 1, 2500])), 0),
    ("long_gqa", dict(S=5, NB=512, lengths=("fixed", [0, 700, 0, 1, 2500])), 512),
    ("long_gqa", dict(S=4, NB=64, bs=8, dtype="f16", lengths=("fixed", [0, 0, 0, 0])), 64),
]


@pytest.mark.parametrize("name,over,part", ZERO_CASES)
def test_zero_length_contexts(name, over, part):
    """Sequences with no tokens get an all-zero output and no stored row;
    the others match the oracle; the fused step equals the two calls bit for
    bit, pools included (an all-empty batch too)."""
    w = synth.make_decode(name, device=DEV, **over)
    alloc = pa.Allocator(w.NB, w.bs, init_order=w.block_order)
    step = np.full(w.S, -1, dtype=np.int64)
    for s in range(w.S):
        alloc.create(s)
        n = int(w.context_lens[s])
        if n:
            slots, _, _ = alloc.append_n(s, n)
            step[s] = slots[-1]
    tables, lens = alloc.build_batch(list(range(w.S)), w.MB)
    assert np.array_equal(tables, w.block_tables) and np.array_equal(lens, w.context_lens)
    mx = max(1, int(lens.max()))
    note(f"case zero-length {name} {over} part={part} lens={lens.tolist()}")
    t_d, l_d = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
    ws = pa.make_workspace(w.S, w.Hq, w.D, mx, part)
    kc1, vc1 = w.key_cache.clone(), w.value_cache.clone()
    out1 = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
    pa.pa_reshape_and_cache(w.new_key, w.new_value, kc1, vc1, torch.from_numpy(step).to(DEV))
    pa.pa_decode_attention(out1, w.q, kc1, vc1, t_d, l_d, mx, w.scale, part, ws)
    kc2, vc2 = w.key_cache.clone(), w.value_cache.clone()
    out2 = torch.full_like(out1, float("nan"))
    pa.pa_decode_step(out2, w.q, w.new_key, w.new_value, kc2, vc2, t_d, l_d, mx, w.scale, part,
                      ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(out2))
    assert torch.equal(bits(kc1), bits(kc2)) and torch.equal(bits(vc1), bits(vc2))
    got = widened(out2, w.dtype)
    empty = [s for s in range(w.S) if lens[s] == 0]
    full = [s for s in range(w.S) if lens[s] > 0]
    assert np.array_equal(got[empty], np.zeros_like(got[empty]))      # exact zeros
    if full:
        ref, oslots = oracle_step(w, full)
        assert np.array_equal(step[full], oslots)
        err = float(np.max(np.abs(got[full] - ref)))
        note(f"  max abs err {err:.3e}")
        assert err <= TOL[w.dtype]


# ---------------------------------------------------------------------------
# the engine (allocator + kernels sequenced in Python) against the oracle's own
# drive of the same shared-prefix script
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("prompt_len", [504, 512])
def test_engine_shared_prefix(prompt_len):
    from paged_kv_cache_198_amd import engine
    sc = synth.make_shared_prefix(device=DEV, prompt_len=prompt_len, prompts=3, NB=512,
                                  tail=(0, 40))
    kv = engine.build_shared_prefix(sc)
    out = kv.step(sc.q, list(range(sc.S)), sc.step_k, sc.step_v, sc.scale)
    torch.cuda.synchronize()
    ref, rkc, rvc, rtables, rlens, _, rexp = drive_shared_prefix_oracle(sc)
    tables, lens, _ = kv.batch(list(range(sc.S)), MB=rtables.shape[1])
    assert np.array_equal(tables.cpu().numpy(), rtables)
    assert np.array_equal(lens.cpu().numpy(), rlens)
    ref_counts, free = kv.alloc.export()
    assert ref_counts == rexp[0] and free == rexp[1]
    assert np.array_equal(synth.to_numpy_storage(kv.key_cache).view(np.uint16), rkc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(kv.value_cache).view(np.uint16), rvc.view(np.uint16))
    err = float(np.max(np.abs(widened(out, sc.dtype) - ref)))
    note(f"  engine shared prefix {prompt_len}: copies {kv.copies}, max abs err {err:.3e}")
    assert err <= TOL[sc.dtype]


# ---------------------------------------------------------------------------
# block sizes 64 and 128 (a 16-token MFMA tile then sits inside one block)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [64, 128])
def test_large_blocks_mha(bs):
    w = synth.make_decode("llama13b", device=DEV, bs=bs, S=6, pool_tokens=32768,
                          lengths=("fixed", [1, 63, 64, 65, 700, 2048]))
    check_decode(w)
    check_decode(w, part=2 * bs)


@pytest.mark.parametrize("bs", [64, 128])
def test_large_blocks_gqa(bs):
    w = synth.make_decode("long_gqa", device=DEV, bs=bs, S=4, NB=1024,
                          lengths=("fixed", [1, 127, 1000, 5000]))
    check_decode(w)
    check_decode(w, part=512)
    out1, kc1, vc1, _ = run_step(w, 512)
    out2, kc2, vc2 = run_fused(w, 512)
    assert torch.equal(bits(out1), bits(out2)) and torch.equal(bits(kc1), bits(kc2))


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode: forked batches planned by pa_cascade_plan;
# the prefix pass reads shared blocks once per group, and the merged result
# must meet the same oracle bound as the plain decode
# ---------------------------------------------------------------------------
CASCADE_CASES = [  # (G, Hkv, bs, dtype, partition, prefix_tokens)
    (8, 4, 16, "bf16", 0, 0), (8, 4, 16, "f16", 512, 64), (1, 8, 16, "f16", 0, 0),
    (1, 8, 16, "bf16", 64, 128), (2, 4, 8, "bf16", 64, 64), (4, 4, 32, "f16", 128, 128),
    (8, 2, 64, "bf16", 256, 64), (1, 4, 128, "bf16", 0, 128), (8, 4, 16, "bf16", 48, 96),
]


def run_cascade(w, lens, part, pfx, fused):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    plan = pa.pa_cascade_plan(w.block_tables, lens, w.bs, w.Hq, w.Hkv, part, pfx)
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    out = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
    ws = pa.make_cascade_workspace(w.S, w.Hq, w.D, plan)
    note(f"  plan: items {plan.n_items} slots {plan.slots_max} suffix parts {plan.suffix_parts} "
         f"prefix rows {plan.prefix_rows} saved rows {plan.saved_rows}")
    pa.pa_decode_cascade(out, w.q, kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                         torch.from_numpy(lens).to(DEV), plan, max(int(lens.max()), 1), w.scale,
                         part, ws, key=w.new_key if fused else None,
                         value=w.new_value if fused else None)
    torch.cuda.synchronize()
    return out, kc, vc, plan


@pytest.mark.parametrize("G,Hkv,bs,dtype,part,pfx", CASCADE_CASES)
def test_cascade_decode(G, Hkv, bs, dtype, part, pfx):
    w = synth.make_forked(0, device=DEV, Hq=G * Hkv, Hkv=Hkv, bs=bs, dtype=dtype)
    note(f"case cascade decode G={G} Hkv={Hkv} bs={bs} {dtype} part={part} prefix={pfx} "
         f"S={w.S} max_ctx={w.max_context_len}")
    lens = np.maximum(w.context_lens - 1, 0).astype(np.int32)   # the pool holds ctx-1 tokens
    out, kc, vc, plan = run_cascade(w, lens, part, pfx, fused=False)
    assert (plan.items[:, 4] > 1).any()                     # some prefix is shared
    live = [s for s in range(w.S) if lens[s] > 0]
    ref, _ = oracle_step(w, live, lens=lens, write=False)
    got = widened(out, w.dtype)
    err = float(np.max(np.abs(got[live] - ref)))
    note(f"  max abs err {err:.3e} (bound {TOL[w.dtype]:g})")
    assert err <= TOL[w.dtype]
    dead = [s for s in range(w.S) if lens[s] == 0]
    assert not got[dead].any()
    # the pools are read only
    assert torch.equal(bits(kc), bits(w.key_cache)) and torch.equal(bits(vc), bits(w.value_cache))


@pytest.mark.parametrize("G,Hkv,bs,dtype,part,pfx", CASCADE_CASES)
def test_cascade_step(G, Hkv, bs, dtype, part, pfx):
    w = synth.make_forked(1, device=DEV, Hq=G * Hkv, Hkv=Hkv, bs=bs, dtype=dtype)
    note(f"case cascade step G={G} Hkv={Hkv} bs={bs} {dtype} part={part} prefix={pfx} "
         f"S={w.S} max_ctx={w.max_context_len}")
    out, kc, vc, plan = run_cascade(w, w.context_lens, part, pfx, fused=True)
    assert (plan.items[:, 4] > 1).any()
    ref, slots = oracle_step(w)
    err = float(np.max(np.abs(widened(out, w.dtype) - ref)))
    note(f"  max abs err {err:.3e} (bound {TOL[w.dtype]:g})")
    assert err <= TOL[w.dtype]
    # pools: the step's rows at the oracle's slots, every other bit unchanged
    ekc, evc = od.reshape_and_cache(synth.to_numpy_storage(w.new_key),
                                    synth.to_numpy_storage(w.new_value),
                                    synth.to_numpy_storage(w.key_cache),
                                    synth.to_numpy_storage(w.value_cache), slots)
    assert np.array_equal(synth.to_numpy_storage(kc).view(np.uint16), ekc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(vc).view(np.uint16), evc.view(np.uint16))


@pytest.mark.parametrize("name,over,part", [
    ("llama13b", dict(S=6, pool_tokens=16384), 0),
    ("llama13b", dict(S=6, pool_tokens=16384), 256),
    ("llama13b", dict(S=6, bs=64, pool_tokens=16384, lengths=("fixed", [1, 63, 64, 65, 700, 2048])), 128),
    ("long_gqa", dict(S=3, NB=1024, lengths=("uniform", 700, 4000)), 512),
    ("long_gqa", dict(S=4, NB=1024, lengths=("fixed", [1, 31, 32, 1025])), 0),
    ("long_gqa", dict(S=3, NB=2048, bs=8, dtype="f16", lengths=("uniform", 1, 3000)), 64),
    ("long_gqa", dict(S=3, NB=2048, lengths=("uniform", 1, 3000)), 48),
])
def test_cascade_without_sharing(name, over, part):
    # no shared blocks: every item is one sequence's partition; the cache
    # write is exact, the output within the oracle bound, and with G = 8 (the
    # plain step on the same matrix-core arithmetic) bit-identical to it
    w = synth.make_decode(name, device=DEV, **over)
    note(f"case cascade no-sharing {name} {over} part={part}")
    out1, kc1, vc1 = run_fused(w, part)
    out2, kc2, vc2, plan = run_cascade(w, w.context_lens, part, 0, fused=True)
    assert not (plan.items[:, 4] > 1).any()
    assert torch.equal(bits(kc1), bits(kc2)) and torch.equal(bits(vc1), bits(vc2))
    ref, _ = oracle_step(w)
    err = float(np.max(np.abs(widened(out2, w.dtype) - ref)))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    if w.Hq // w.Hkv == 8:
        assert torch.equal(bits(out1), bits(out2))


@pytest.mark.parametrize("full", [False, True])
def test_engine_shared_prefix_cascade(full):
    from paged_kv_cache_198_amd import engine
    kw = dict(prompt_len=504) if full else dict(prompt_len=512, prompts=3, NB=512, tail=(0, 40))
    sc = synth.make_shared_prefix(device=DEV, **kw)
    note(f"case engine cascade prompts={sc.prompts} S={sc.S} prompt_len={sc.prompt_len}")
    kv = engine.build_shared_prefix(sc)
    out, plan = kv.step_cascade(sc.q, list(range(sc.S)), sc.step_k, sc.step_v, sc.scale,
                                prefix_tokens=128)
    torch.cuda.synchronize()
    ref, rkc, rvc, rtables, rlens, _, _ = drive_shared_prefix_oracle(sc)
    # every sample shares its prompt's full blocks (rounded to 32 tokens)
    assert (plan.seq_start == (sc.prompt_len // sc.bs * sc.bs) // 32 * 32).all()
    assert np.array_equal(synth.to_numpy_storage(kv.key_cache).view(np.uint16), rkc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(kv.value_cache).view(np.uint16), rvc.view(np.uint16))
    err = float(np.max(np.abs(widened(out, sc.dtype) - ref)))
    note(f"  engine cascade: items {plan.n_items}, saved rows {plan.saved_rows}, "
         f"max abs err {err:.3e}")
    assert err <= TOL[sc.dtype]


# ---------------------------------------------------------------------------
# sharing across requests: a system prompt registered once and reused by
# later requests through the prefix registry, decoded plain and as a cascade,
# against the oracle allocator's own drive of the same script
# ---------------------------------------------------------------------------
def drive_system_prompt_oracle(sc):
    kc = synth.to_numpy_storage(sc.key_cache)
    vc = synth.to_numpy_storage(sc.value_cache)
    alloc = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    keys = sc.system_keys()
    for r in range(sc.requests):
        k, v = (synth.to_numpy_storage(t) for t in sc.prompt(r))
        if r == 0:
            alloc.create(0)
            m = 0
        else:
            m = alloc.create_prefixed(r, keys) * sc.bs
        slots = [alloc.append(r)[0] for _ in range(k.shape[0] - m)]
        od.reshape_and_cache(k[m:], v[m:], kc, vc, slots, inplace=True)
        if r == 0:
            alloc.publish(0, keys)
    step = [alloc.append(r) for r in range(sc.requests)]
    assert all(c[1:] == (-1, -1) for c in step)
    od.reshape_and_cache(synth.to_numpy_storage(sc.step_k), synth.to_numpy_storage(sc.step_v),
                         kc, vc, [c[0] for c in step], inplace=True)
    MB = max(len(alloc.table(r)) for r in range(sc.requests))
    tables, lens = alloc.build_batch(list(range(sc.requests)), MB)
    out = od.paged_decode(synth.to_numpy_storage(sc.q), kc, vc, np.array(tables), np.array(lens),
                          sc.scale, sc.dtype)
    return out, kc, vc, np.array(tables), np.array(lens), (list(alloc.ref), alloc.free_stack())


@pytest.mark.parametrize("over", [
    dict(requests=6, NB=512, system_len=100, own=(1, 40)),
    dict(requests=20, NB=1024, system_len=256, own=(16, 200), dtype="f16", Hq=32, Hkv=8),
    dict(requests=9, NB=1024, system_len=300, own=(1, 100), bs=32, Hq=16, Hkv=8),
])
@pytest.mark.parametrize("cascade", [False, True])
def test_system_prompt_shared_across_requests(over, cascade):
    from paged_kv_cache_198_amd import engine
    sc = synth.make_system_prompt(device=DEV, **over)
    note(f"case system prompt {over} cascade={cascade}")
    kv = engine.build_system_prompt(sc)
    ids = list(range(sc.requests))
    if cascade:
        out, plan = kv.step_cascade(sc.q, ids, sc.step_k, sc.step_v, sc.scale, prefix_tokens=64)
    else:
        out = kv.step(sc.q, ids, sc.step_k, sc.step_v, sc.scale)
    torch.cuda.synchronize()
    ref, rkc, rvc, rtables, rlens, rexp = drive_system_prompt_oracle(sc)
    tables, lens, _ = kv.batch(ids, MB=rtables.shape[1])
    assert np.array_equal(tables.cpu().numpy(), rtables) and np.array_equal(lens.cpu().numpy(), rlens)
    ref_counts, free = kv.alloc.export()
    assert ref_counts == rexp[0] and free == rexp[1]
    assert np.array_equal(synth.to_numpy_storage(kv.key_cache).view(np.uint16), rkc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(kv.value_cache).view(np.uint16), rvc.view(np.uint16))
    # the system prompt is stored once
    n_sys = sc.system_len // sc.bs
    assert kv.used_blocks() == n_sys + sum(-(-(sc.system_len + 1 + int(n)) // sc.bs) - n_sys
                                           for n in sc.own_lens)
    if cascade:
        # requests in chunks of 16/G; a last chunk of one shares nothing
        per = 16 // (sc.Hq // sc.Hkv)
        chunks = sc.requests // per + (1 if sc.requests % per >= 2 else 0)
        grouped = sc.requests - (1 if sc.requests % per == 1 else 0)
        T_sh = n_sys * sc.bs // max(32, sc.bs) * max(32, sc.bs)
        assert int((plan.seq_start == T_sh).sum()) == grouped
        assert int((plan.items[:, 4] > 1).sum()) == chunks * -(-T_sh // 64)
    err = float(np.max(np.abs(widened(out, sc.dtype) - ref)))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[sc.dtype]


# ---------------------------------------------------------------------------
# beam search: forks and discards every step, copy-on-write copies batched
# across all layers, several layers sharing one block table per sequence
# ---------------------------------------------------------------------------
def drive_beam_lib(sc, cascade):
    from paged_kv_cache_198_amd import engine
    kv = engine.PagedKV(sc.NB, sc.bs, sc.Hkv, sc.D, sc.dtype, init_order=sc.init_order,
                        device=DEV, layers=sc.layers)
    for i in range(sc.layers):
        kv.key_caches[i].copy_(sc.key_cache)
        kv.value_caches[i].copy_(sc.value_cache)
    beams, nxt = [], sc.requests
    for r in range(sc.requests):
        kv.prefill(r, sc.prompt_k[r], sc.prompt_v[r])
        group = [r]
        for _ in range(sc.width - 1):
            kv.fork(r, nxt)
            group.append(nxt)
            nxt += 1
        beams.append(group)
    log = []
    for t in range(sc.steps):
        beams, nxt = engine.beam_reselect(kv, beams, sc.choices[t].tolist(), nxt)
        flat = [b for g in beams for b in g]
        if t < sc.steps - 1:
            slots, pairs = kv.append(flat, sc.step_k[t], sc.step_v[t])
            log.append((slots.tolist(), pairs))
    before = kv.copies
    if cascade:
        out, plan = kv.step_cascade(sc.q, flat, sc.step_k[-1], sc.step_v[-1], sc.scale)
    else:
        out = kv.step(sc.q, flat, sc.step_k[-1], sc.step_v[-1], sc.scale)
    torch.cuda.synchronize()
    return kv, flat, out, log, kv.copies - before


def drive_beam_oracle(sc):
    L = sc.layers
    kc = [synth.to_numpy_storage(sc.key_cache) for _ in range(L)]
    vc = [synth.to_numpy_storage(sc.value_cache) for _ in range(L)]
    alloc = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    beams, nxt = [], sc.requests
    for r in range(sc.requests):
        alloc.create(r)
        n = int(sc.prompt_lens[r])
        slots = [alloc.append(r)[0] for _ in range(n)]
        pk, pv = synth.to_numpy_storage(sc.prompt_k[r]), synth.to_numpy_storage(sc.prompt_v[r])
        for i in range(L):
            od.reshape_and_cache(pk[i], pv[i], kc[i], vc[i], slots, inplace=True)
        group = [r]
        for _ in range(sc.width - 1):
            alloc.fork(r, nxt)
            group.append(nxt)
            nxt += 1
        beams.append(group)
    sk, sv = synth.to_numpy_storage(sc.step_k), synth.to_numpy_storage(sc.step_v)
    log = []
    for t in range(sc.steps):
        new = []
        for cur, pick in zip(beams, sc.choices[t].tolist()):
            used, nb = set(), []
            for i in pick:
                if i not in used:
                    used.add(i)
                    nb.append(cur[i])
                else:
                    alloc.fork(cur[i], nxt)
                    nb.append(nxt)
                    nxt += 1
            for i, sid in enumerate(cur):
                if i not in used:
                    alloc.release(sid)
            new.append(nb)
        beams = new
        flat = [b for g in beams for b in g]
        res = [alloc.append(b) for b in flat]
        slots = [x[0] for x in res]
        pairs = [(x[1], x[2]) for x in res if x[1] >= 0]
        od.copy_blocks(kc, vc, pairs, inplace=True)
        for i in range(L):
            od.reshape_and_cache(sk[t, i], sv[t, i], kc[i], vc[i], slots, inplace=True)
        if t < sc.steps - 1:
            log.append((slots, pairs))
        else:
            last_pairs = len(pairs)
    MB = max(len(alloc.table(b)) for b in flat)
    tables, lens = alloc.build_batch(flat, MB)
    q = synth.to_numpy_storage(sc.q)
    outs = [od.paged_decode(q[i], kc[i], vc[i], np.array(tables), np.array(lens), sc.scale,
                            sc.dtype) for i in range(L)]
    return (flat, np.stack(outs), kc, vc, np.array(tables), np.array(lens), log, last_pairs,
            (list(alloc.ref), alloc.free_stack()))


@pytest.mark.parametrize("over,cascade", [
    ({}, False), ({}, True),
    (dict(bs=16, dtype="f16", Hq=32, Hkv=4, steps=20, requests=2, width=6), False),
    (dict(bs=16, dtype="f16", Hq=32, Hkv=4, steps=20, requests=2, width=6), True),
    (dict(bs=32, Hq=4, Hkv=4, layers=2, width=8, steps=40, prompt=(20, 70)), True),
])
def test_beam_search_churn(over, cascade):
    sc = synth.make_beam(device=DEV, **over)
    note(f"case beam {over} cascade={cascade}")
    kv, flat, out, log, last_copies = drive_beam_lib(sc, cascade)
    rflat, ref, rkc, rvc, rtables, rlens, rlog, rlast, rexp = drive_beam_oracle(sc)
    assert flat == rflat
    assert log == rlog                                    # slots and copy pairs, every step
    assert last_copies == rlast
    tables, lens, _ = kv.batch(flat, MB=rtables.shape[1])
    assert np.array_equal(tables.cpu().numpy(), rtables) and np.array_equal(lens.cpu().numpy(), rlens)
    assert kv.alloc.export() == (rexp[0], rexp[1])
    for i in range(sc.layers):                            # every layer's pools, bit for bit
        assert np.array_equal(synth.to_numpy_storage(kv.key_caches[i]).view(np.uint16),
                              rkc[i].view(np.uint16))
        assert np.array_equal(synth.to_numpy_storage(kv.value_caches[i]).view(np.uint16),
                              rvc[i].view(np.uint16))
    copies = sum(len(p) for _, p in log) + last_copies
    err = float(np.max(np.abs(widened(out, sc.dtype) - ref)))
    note(f"  copies {copies}, max abs err {err:.3e}")
    assert copies > 0
    assert err <= TOL[sc.dtype]


# ---------------------------------------------------------------------------
# paged prefill attention: chunks of new tokens stored with
# pa_reshape_and_cache, then attended causally (matrix cores)
# ---------------------------------------------------------------------------
def prefill_bound(ref, dtype):
    """Per-element bound for prefill outputs.  The stated bound (1e-2 bf16,
    2e-3 f16) holds while the output's own rounding stays below it, which for
    bf16 means |out| < 4; rows near a prompt's start average few values and
    can exceed that, and there no bf16 result can be closer than half an ulp
    (0.0156 in [4, 8)).  So the bound is max(stated, 1.25 half-ulps of the
    reference in the KV type)."""
    bits = {"bf16": 8, "f16": 11, "f32": 24}[dtype]
    a = np.maximum(np.abs(ref), 1e-30)
    half_ulp = np.exp2(np.floor(np.log2(a)) - bits)
    return np.maximum(TOL[dtype], 1.25 * half_ulp)


def run_prefill_lib(w, context_lens=None, max_query_len=None):
    lens = w.context_lens if context_lens is None else np.asarray(context_lens, dtype=np.int32)
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    if w.T:
        pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc,
                                torch.from_numpy(lib_prefill_slots(w)).to(DEV))
    out = torch.full((max(w.T, 1), w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)[:w.T]
    mq = int(w.chunk_lens.max()) if max_query_len is None else max_query_len
    pa.pa_prefill_attention(out, w.q, kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                            torch.from_numpy(lens).to(DEV),
                            torch.from_numpy(w.query_start).to(DEV), mq, w.scale)
    torch.cuda.synchronize()
    return out, kc, vc


def prefill_oracle(w, context_lens=None, seqs=None):
    lens = w.context_lens if context_lens is None else np.asarray(context_lens)
    kc, vc = od.reshape_and_cache(synth.to_numpy_storage(w.new_key),
                                  synth.to_numpy_storage(w.new_value),
                                  synth.to_numpy_storage(w.key_cache),
                                  synth.to_numpy_storage(w.value_cache),
                                  oracle_prefill_slots(w))
    out = od.paged_prefill(synth.to_numpy_storage(w.q), kc, vc, w.block_tables, lens,
                           w.query_start, w.scale, w.dtype, seqs=seqs)
    return out, kc, vc


PREFILL_CASES = [  # (G, Hkv, bs, dtype, prefix law, chunk law)
    (1, 4, 16, "bf16", ("fixed", 0), ("uniform", 1, 200)),
    (1, 4, 16, "f16", ("uniform", 0, 300), ("uniform", 1, 150)),
    (2, 4, 8, "bf16", ("uniform", 0, 200), ("uniform", 1, 100)),
    (4, 2, 32, "f16", ("uniform", 1, 400), ("uniform", 1, 70)),
    (8, 2, 64, "bf16", ("uniform", 0, 700), ("uniform", 1, 90)),
    (8, 4, 128, "bf16", ("fixed", 0), ("fixed", [1, 2, 31, 32, 33, 64])),
    (1, 2, 128, "f16", ("fixed", [0, 127, 128, 129, 5, 1000]), ("fixed", [0, 1, 64, 65, 300, 7])),
    # query tiles of 64 rows (G = 2) cut just before, at and after their end;
    # key ranges ending off the 64-key stages
    (2, 3, 16, "bf16", ("fixed", [0, 63, 64, 65, 1, 190]), ("fixed", [63, 64, 65, 127, 128, 129])),
    (4, 2, 128, "f16", ("fixed", [33, 0, 191, 64, 250, 3]), ("fixed", [31, 32, 33, 96, 5, 200])),
    (1, 1, 8, "bf16", ("fixed", [7, 8, 9, 56, 57, 500]), ("fixed", [121, 8, 199, 1, 72, 13])),
]


@pytest.mark.parametrize("G,Hkv,bs,dtype,prefix,chunk", PREFILL_CASES)
def test_prefill_against_oracle(G, Hkv, bs, dtype, prefix, chunk):
    S = len(chunk[1]) if chunk[0] == "fixed" and np.ndim(chunk[1]) else 6
    w = synth.make_prefill(0, device=DEV, S=S, Hq=G * Hkv, Hkv=Hkv, bs=bs, dtype=dtype,
                           pool_tokens=32768, prefix=prefix, chunk=chunk)
    note(f"case prefill G={G} Hkv={Hkv} bs={bs} {dtype} chunks={w.chunk_lens.tolist()} "
         f"ctx={w.context_lens.tolist()}")
    assert np.array_equal(lib_prefill_slots(w), oracle_prefill_slots(w))   # slots bit-exact
    out, kc, vc = run_prefill_lib(w)
    ref, rkc, rvc = prefill_oracle(w)
    assert np.array_equal(synth.to_numpy_storage(kc).view(np.uint16), rkc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(vc).view(np.uint16), rvc.view(np.uint16))
    got = widened(out, w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref))) if w.T else 0.0
    note(f"  max abs err {err:.3e}, max |ref| {float(np.max(np.abs(ref))) if w.T else 0:.2f}")
    assert (np.abs(got - ref) <= prefill_bound(ref, w.dtype)).all()


def test_prefill_edges():
    # chunks longer than the context (rows before position 0 are zero), a
    # sequence with no chunk, and a grid bound tighter than one chunk: rows
    # past the bound are left untouched
    w = synth.make_prefill(1, device=DEV, S=4, Hq=8, Hkv=4, bs=16, pool_tokens=8192,
                           prefix=("fixed", [0, 10, 0, 3]), chunk=("fixed", [20, 0, 5, 80]))
    lens = w.context_lens.copy()
    lens[0] = 12                        # 20 rows, 12 keys: the first 8 rows see nothing
    out, _, _ = run_prefill_lib(w, context_lens=lens)
    ref, _, _ = prefill_oracle(w, context_lens=lens)
    got = widened(out, w.dtype)
    assert not got[:8].any()
    assert (np.abs(got - ref) <= prefill_bound(ref, w.dtype)).all()
    out2, _, _ = run_prefill_lib(w, max_query_len=16)
    got2 = widened(out2, w.dtype)
    qs = w.query_start
    # G = 2: a tile holds 8 wavefronts x 8 = 64 query rows, tiles start at
    # multiples of 64 and run last first, so one launched tile covers
    # sequence 3's rows 64..79 of 80
    assert np.isnan(got2[qs[3]:qs[3] + 64]).all()
    ref2, _, _ = prefill_oracle(w)
    for a, b in ((qs[3] + 64, qs[4]), (0, qs[3])):
        assert (np.abs(got2[a:b] - ref2[a:b]) <= prefill_bound(ref2[a:b], w.dtype)).all()


def test_prefill_table_entry_outside_pool():
    # an entry outside [0, NB) inside a context is never dereferenced; its
    # tokens take part as zero keys and values (the oracle sees the same
    # entry pointing at an all-zero block appended to its pool)
    w = synth.make_prefill(2, device=DEV, S=3, Hq=8, Hkv=8, bs=16, pool_tokens=4096,
                           prefix=("fixed", [40, 0, 70]), chunk=("fixed", [20, 50, 9]))
    bad = w.block_tables.copy()
    bad[0, 1] = w.NB + 3
    bad[2, 0] = -7
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc,
                            torch.from_numpy(lib_prefill_slots(w)).to(DEV))
    out = torch.empty_like(w.q)
    pa.pa_prefill_attention(out, w.q, kc, vc, torch.from_numpy(bad).to(DEV),
                            torch.from_numpy(w.context_lens).to(DEV),
                            torch.from_numpy(w.query_start).to(DEV), int(w.chunk_lens.max()),
                            w.scale)
    torch.cuda.synchronize()
    okc = synth.to_numpy_storage(kc)
    ovc = synth.to_numpy_storage(vc)
    zero = np.zeros((1,) + okc.shape[1:], dtype=okc.dtype)
    okc, ovc = np.concatenate([okc, zero]), np.concatenate([ovc, zero])
    tab = bad.copy()
    tab[0, 1] = tab[2, 0] = w.NB
    ref = od.paged_prefill(synth.to_numpy_storage(w.q), okc, ovc, tab, w.context_lens,
                           w.query_start, w.scale, w.dtype)
    got = widened(out, w.dtype)
    assert (np.abs(got - ref) <= prefill_bound(ref, w.dtype)).all()


def test_prefill_full_size_sampled():
    w = synth.make_prefill(0, device=DEV)
    note(f"case prefill full: S={w.S} T={w.T} max chunk {int(w.chunk_lens.max())}")
    out, _, _ = run_prefill_lib(w)
    seqs = [int(np.argmax(w.chunk_lens)), int(np.argmin(w.chunk_lens)), 3]
    ref, _, _ = prefill_oracle(w, seqs=seqs)
    got = widened(out, w.dtype)
    assert np.isfinite(got).all()
    for s in seqs:
        r0, r1 = w.query_start[s], w.query_start[s + 1]
        err = float(np.max(np.abs(got[r0:r1] - ref[r0:r1])))
        note(f"  sequence {s} ({r1 - r0} rows): max abs err {err:.3e}")
        assert (np.abs(got[r0:r1] - ref[r0:r1]) <= prefill_bound(ref[r0:r1], w.dtype)).all()


def test_engine_chunked_prefill_with_registry():
    """Request 0 prefills its prompt in two chunks; request 1 takes the
    system prompt's blocks from the registry and prefills only its own
    tokens; request 2 is forked from request 0 mid-block and continues with a
    chunk (its first append copies the shared block).  Every chunk's output
    against the oracle's prefill over the oracle's own pool and tables."""
    from paged_kv_cache_198_amd import engine
    sc = synth.make_system_prompt(device=DEV, requests=3, NB=256, system_len=72, own=(20, 60),
                                  Hq=16, Hkv=4, dtype="bf16")
    keys = sc.system_keys()
    kv = engine.PagedKV(sc.NB, sc.bs, sc.Hkv, sc.D, sc.dtype, init_order=sc.init_order,
                        device=DEV, key_cache=sc.key_cache.clone(),
                        value_cache=sc.value_cache.clone())
    oa_ = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    okc, ovc = synth.to_numpy_storage(sc.key_cache), synth.to_numpy_storage(sc.value_cache)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)

    def chunk_inputs(n):
        q = torch.randn(n, sc.Hq, sc.D, generator=gen, device=DEV).to(sc.q.dtype)
        return q

    def oracle_chunk(sid, k, v, q):
        n = k.shape[0]
        sl = []
        for _ in range(n):
            slot, src, dst = oa_.append(sid)
            if src >= 0:
                od.copy_blocks([okc], [ovc], [(src, dst)], inplace=True)
            sl.append(slot)
        od.reshape_and_cache(synth.to_numpy_storage(k), synth.to_numpy_storage(v), okc, ovc, sl,
                             inplace=True)
        t = np.array([oa_.table(sid)], dtype=np.int32)
        return od.paged_prefill(synth.to_numpy_storage(q), okc, ovc, t,
                                np.array([oa_.seq_len(sid)]), np.array([0, n]), sc.scale,
                                sc.dtype)

    def check(got, ref):
        g = widened(got, sc.dtype)
        assert (np.abs(g - ref) <= prefill_bound(ref, sc.dtype)).all()

    k0, v0 = sc.prompt(0)
    T0 = k0.shape[0]
    cut = 40                                        # two chunks, the first ends mid-block
    kv.alloc.create(0)
    oa_.create(0)
    for a, b in ((0, cut), (cut, T0)):
        q = chunk_inputs(b - a)
        out = kv.prefill_chunks([0], [b - a], q, k0[a:b].contiguous(), v0[a:b].contiguous(),
                                sc.scale)
        check(out, oracle_chunk(0, k0[a:b], v0[a:b], q))
    assert kv.publish(0, keys) == oa_.publish(0, keys) == len(keys)
    # request 1: system prompt from the registry, own tokens prefilled
    k1, v1 = sc.prompt(1)
    m = kv.alloc.create_prefixed(1, keys) * sc.bs
    assert m == oa_.create_prefixed(1, keys) * sc.bs == len(keys) * sc.bs
    q = chunk_inputs(k1.shape[0] - m)
    out = kv.prefill_chunks([1], [k1.shape[0] - m], q, k1[m:].contiguous(), v1[m:].contiguous(),
                            sc.scale)
    check(out, oracle_chunk(1, k1[m:], v1[m:], q))
    # request 2: a fork of request 0 continuing with its own chunk
    kv.fork(0, 2)
    oa_.fork(0, 2)
    k2 = torch.randn(30, sc.Hkv, sc.D, generator=gen, device=DEV).to(sc.q.dtype)
    v2 = torch.randn(30, sc.Hkv, sc.D, generator=gen, device=DEV).to(sc.q.dtype)
    q = chunk_inputs(30)
    before = kv.copies
    out = kv.prefill_chunks([2], [30], q, k2, v2, sc.scale)
    check(out, oracle_chunk(2, k2, v2, q))
    assert kv.copies - before == (1 if T0 % sc.bs else 0)
    torch.cuda.synchronize()
    assert np.array_equal(synth.to_numpy_storage(kv.key_cache).view(np.uint16), okc.view(np.uint16))
    assert np.array_equal(synth.to_numpy_storage(kv.value_cache).view(np.uint16), ovc.view(np.uint16))
    assert kv.alloc.export() == (list(oa_.ref), oa_.free_stack())


@pytest.mark.parametrize("extra,grid", [(0, 4096), (3, 4096), (3, 256), (3, 16)])
def test_read_probe_reads_every_chunk(extra, grid):
    # 1 MiB (+ extra 16-byte chunks, a slice cut short) with `grid`
    # workgroups: workgroup b reads the 32 KB slices b, b + grid, ...; thread
    # t of it reads chunks slice + 256 u + t (u = 0..7) of each and stores the
    # XOR of all their words (grid 16: several slices per workgroup)
    n16 = (1 << 16) + extra
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), generator=g, device=DEV, dtype=torch.int32)
    out = torch.full((grid * 256,), -1, dtype=torch.int32, device=DEV)
    pa.pa_probe_read_bandwidth(src, out)
    torch.cuda.synchronize()
    w = src.cpu().numpy().view(np.uint32).reshape(-1, 4)
    fold = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    slices = -(-n16 // 2048)
    padded = np.zeros(slices * 2048, dtype=np.uint32)
    padded[:n16] = fold
    per_slice = np.bitwise_xor.reduce(padded.reshape(slices, 8, 256), axis=1)
    expect = np.zeros((grid, 256), dtype=np.uint32)
    for k in range(slices):
        expect[k % grid] ^= per_slice[k]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), expect.reshape(-1))


# ---------------------------------------------------------------------------
# seeded random configurations: dtype, head dim, group size, KV heads, block
# size, ragged lengths and partition size drawn together, through both the
# fused step and the two-call path
# ---------------------------------------------------------------------------
def _random_config(i):
    import random
    r = random.Random(7000 + i)
    dtype = r.choice(["f32", "f16", "bf16"])
    D = r.choice([64, 128])
    G = r.choice([1, 2, 4, 8])
    Hkv = r.choice([1, 2, 3, 4])
    bs = r.choice([8, 16, 32, 64, 128])
    S = r.randint(1, 6)
    hi = r.choice([40, 300, 1500, 4000])
    lens = [r.randint(1, hi) for _ in range(S)]
    NB = max(64, sum(-(-n // bs) for n in lens) + r.randint(0, 64))
    part = r.choice([0, bs * r.randint(1, 8), (32 if bs <= 32 else bs) * r.randint(1, 16)])
    return dtype, D, G, Hkv, bs, lens, NB, part


@pytest.mark.parametrize("i", range(16))
def test_random_configurations(i):
    dtype, D, G, Hkv, bs, lens, NB, part = _random_config(i)
    note(f"case random {i}: {dtype} D={D} G={G} Hkv={Hkv} bs={bs} lens={lens} NB={NB} part={part}")
    w = synth.make_decode("llama7b", device=DEV, S=len(lens), Hq=Hkv * G, Hkv=Hkv, D=D,
                          dtype=dtype, bs=bs, NB=NB, lengths=("fixed", lens), seed=8000 + i)
    ref, _ = oracle_step(w)
    out1, _, _, _ = run_step(w, part)
    out2, _, _ = run_fused(w, part)
    assert torch.equal(bits(out1), bits(out2))
    err = float(np.max(np.abs(widened(out1, dtype) - ref)))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[dtype]
