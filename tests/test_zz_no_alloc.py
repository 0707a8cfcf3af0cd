"""pa_decode_step_noalloc against pa_decode_step (GPU, through the C ABI).

The no-alloc step runs the same kernels with the split-context partials in
the library's static per-GPU scratch instead of a caller workspace, so its
outputs and pools must equal pa_decode_step's bit for bit.  Two calls in a
row, the second on a smaller input (the scratch keeps the first call's
partials, which must not matter), then a shape that needs no workspace; and
a request larger than the scratch is refused before anything is enqueued.
"""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_198_amd as pa
from paged_kv_cache_198_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def tables_and_lens(w):
    alloc = pa.Allocator(w.NB, w.bs, init_order=w.block_order)
    for s in range(w.S):
        alloc.create(s)
        alloc.append_n(s, int(w.context_lens[s]))
    tables, lens = alloc.build_batch(list(range(w.S)), w.MB)
    assert np.array_equal(tables, w.block_tables)
    return torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)


def both(w, part):
    """(out, K pool, V pool) of pa_decode_step with its own workspace and of
    pa_decode_step_noalloc, from the same pre-step pools."""
    tables, lens = tables_and_lens(w)
    mx = w.max_context_len
    need = pa.pa_decode_workspace_bytes(w.S, w.Hq, w.D, mx, part)
    note(f"case no-alloc {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} bs={w.bs} {w.dtype} "
         f"part={part} max_ctx={mx} workspace={need} B")
    assert need <= pa.PA_STATIC_SCRATCH_BYTES
    res = []
    for noalloc in (False, True):
        kc, vc = w.key_cache.clone(), w.value_cache.clone()
        out = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=w.q.dtype, device=DEV)
        if noalloc:
            pa.pa_decode_step_noalloc(out, w.q, w.new_key, w.new_value, kc, vc, tables, lens, mx,
                                      w.scale, part)
        else:
            ws = pa.make_workspace(w.S, w.Hq, w.D, mx, part)
            pa.pa_decode_step(out, w.q, w.new_key, w.new_value, kc, vc, tables, lens, mx, w.scale,
                              part, ws)
        torch.cuda.synchronize()
        res.append((out, kc, vc))
    return res


def assert_same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(bits(x), bits(y))


def test_noalloc_equals_decode_step_twice():
    # 1: grouped heads on the matrix cores, up to 24 partitions (wide reduce)
    big = synth.make_decode("long_gqa", device=DEV, S=4, NB=4096,
                            lengths=("uniform", 3000, 12000))
    ref, got = both(big, 512)
    assert_same(ref, got)
    # 2: a smaller batch on the vector ALUs right after, 2-5 partitions
    small = synth.make_decode("llama13b", device=DEV, S=3, bs=16, pool_tokens=8192,
                              lengths=("uniform", 300, 1200))
    ref2, got2 = both(small, 256)
    assert_same(ref2, got2)
    assert np.isfinite(got2[0].float().cpu().numpy()).all()
    # 3: one pass, no partials at all
    tiny = synth.make_decode("tiny", device=DEV)
    ref3, got3 = both(tiny, 0)
    assert_same(ref3, got3)


def test_noalloc_refuses_more_than_the_scratch():
    w = synth.make_decode("tiny", device=DEV)
    tables, lens = tables_and_lens(w)
    out = torch.empty(w.S, w.Hq, w.D, dtype=w.q.dtype, device=DEV)
    kc = w.key_cache.clone()
    before = bits(kc).clone()
    # max_context_len far above the table's reach is capped at MB*bs; a
    # 16-token partition of a 64-block table still fits, so widen the table
    wide = torch.full((w.S, 8192), -1, dtype=torch.int32, device=DEV)
    wide[:, :tables.shape[1]] = tables
    need = pa.pa_decode_workspace_bytes(w.S, w.Hq, w.D, 8192 * w.bs, 16)
    assert need > pa.PA_STATIC_SCRATCH_BYTES
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_step_noalloc(out, w.q, w.new_key, w.new_value, kc, w.value_cache.clone(),
                                  wide, lens, 8192 * w.bs, w.scale, 16)
    assert e.value.status == pa.PA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.equal(bits(kc), before)           # nothing was enqueued


def test_noalloc_full_long_context_batch():
    # the largest workload's partials (8 sequences x 64 query heads, contexts
    # up to 32k tokens in 512-token partitions: 17 MB) fit the static scratch
    w = synth.make_decode("long_gqa", device=DEV)
    ref, got = both(w, w.partition_tokens)
    assert_same(ref, got)
