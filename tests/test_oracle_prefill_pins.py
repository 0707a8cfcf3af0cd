"""Pins for the prefill oracle, ``oracle.decode.paged_prefill`` (CPU only).

Causal attention over a chunk of new tokens whose keys and values sit in the
paged pool ("PagedAttention: the KV cache was the bottleneck all along",
section "Virtual memory for attention": prompt tokens fill blocks acquired as
the sequence grows, and attention gathers them through the block table).
Each pin checks it against something other than itself: torch's
``scaled_dot_product_attention`` in float64 on a separately built contiguous
store (its own causal mask for whole prompts, an explicit offset mask for
chunks), the already pinned decode oracle for a chunk's last row, closed
forms, and invariances of the causal rule (chunking, grouped heads).
``test_oracle_mutants.py`` plants mistakes and checks these pins catch them.
"""
import numpy as np
import pytest
import torch

import oracle.decode as od
from test_oracle_pins import contiguous_store, page_out


def packed(rng, ns, Hq, D):
    """Queries for chunks of ``ns`` tokens, packed, and the row offsets."""
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float32)
    return q, qs


def sdpa_chunk(q_rows, K, V, scale, ctx, G, causal_flag):
    """torch SDPA, float64: queries are the last len(q_rows) positions of a
    ctx-token sequence."""
    n = q_rows.shape[0]
    qt = torch.from_numpy(q_rows.astype(np.float64)).permute(1, 0, 2)         # [Hq, n, D]
    k = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    v = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    sc = float(np.float32(scale))
    if causal_flag:               # n == ctx: the library's own causal mask
        o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=sc)
    else:
        pos = torch.arange(ctx - n, ctx)[:, None]
        mask = torch.arange(ctx)[None, :] <= pos                               # [n, ctx]
        o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=sc)
    return o.permute(1, 0, 2).numpy()


def pin_prefill_sdpa(seed=21):
    rng = np.random.default_rng(seed)
    for Hq, Hkv, bs in ((4, 4, 16), (8, 2, 8), (6, 3, 32)):
        D = 16
        lens = [1, 7, 33, 64, 90]
        ns = [1, 7, 20, 64, 5]                         # whole prompts and chunks
        Ks, Vs = contiguous_store(rng, lens, Hkv, D)
        kc, vc, tables = page_out(Ks, Vs, bs, 64, rng)
        q, qs = packed(rng, ns, Hq, D)
        scale = 0.37
        out = od.paged_prefill(q, kc, vc, tables, np.array(lens), qs, scale, "f32")
        for s, (n, ctx) in enumerate(zip(ns, lens)):
            ref = sdpa_chunk(q[qs[s]:qs[s + 1]], Ks[s], Vs[s], scale, ctx, Hq // Hkv, n == ctx)
            assert np.allclose(out[qs[s]:qs[s + 1]], ref, atol=1e-12, rtol=0)


def pin_prefill_last_row_is_decode(seed=22):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 8, 4, 16, 16
    lens, ns = [5, 40, 77], [5, 3, 30]
    Ks, Vs = contiguous_store(rng, lens, Hkv, D)
    kc, vc, tables = page_out(Ks, Vs, bs, 32, rng)
    q, qs = packed(rng, ns, Hq, D)
    out = od.paged_prefill(q, kc, vc, tables, np.array(lens), qs, 0.25, "f32")
    last = q[qs[1:] - 1]
    dec = od.paged_decode(last, kc, vc, tables, np.array(lens), 0.25, "f32")
    assert np.allclose(out[qs[1:] - 1], dec, atol=1e-13, rtol=0)


def pin_prefill_chunking(seed=23):
    """One chunk of n tokens equals the same tokens split into two chunks,
    each attending the pool with the context it has at that point."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 4, 2, 16, 8
    ctx = 70
    Ks, Vs = contiguous_store(rng, [ctx], Hkv, D)
    kc, vc, tables = page_out(Ks, Vs, bs, 16, rng)
    q = rng.standard_normal((50, Hq, D)).astype(np.float32)       # positions 20 .. 69
    whole = od.paged_prefill(q, kc, vc, tables, np.array([ctx]), np.array([0, 50]), 0.3, "f32")
    a = od.paged_prefill(q[:18], kc, vc, tables, np.array([38]), np.array([0, 18]), 0.3, "f32")
    b = od.paged_prefill(q[18:], kc, vc, tables, np.array([ctx]), np.array([0, 32]), 0.3, "f32")
    assert np.allclose(whole, np.concatenate([a, b]), atol=1e-14, rtol=0)


def pin_prefill_closed_forms(seed=24):
    rng = np.random.default_rng(seed)
    Hkv, D, bs, ctx = 2, 8, 4, 13
    k = np.tile(rng.standard_normal((1, Hkv, D)).astype(np.float32), (ctx, 1, 1))   # equal keys
    v = rng.standard_normal((ctx, Hkv, D)).astype(np.float32)
    kc, vc, tables = page_out([k], [v], bs, 8, rng)
    q = rng.standard_normal((ctx, Hkv, D)).astype(np.float32)
    out = od.paged_prefill(q, kc, vc, tables, np.array([ctx]), np.array([0, ctx]), 0.5, "f32")
    # equal keys: token p's output is the mean of values 0..p
    running = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, ctx + 1)[:, None, None]
    assert np.allclose(out, running, atol=1e-13, rtol=0)
    # the first token of a prompt sees only itself: its value row
    assert np.allclose(out[0], v[0], atol=1e-15, rtol=0)


def pin_prefill_overlong_chunk(seed=25):
    """A chunk longer than the context: rows before position 0 are zero, the
    rest equal the chunk of exactly ctx tokens."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs, ctx = 4, 4, 8, 8, 10
    Ks, Vs = contiguous_store(rng, [ctx], Hkv, D)
    kc, vc, tables = page_out(Ks, Vs, bs, 4, rng)
    q = rng.standard_normal((14, Hq, D)).astype(np.float32)
    long = od.paged_prefill(q, kc, vc, tables, np.array([ctx]), np.array([0, 14]), 0.4, "f32")
    exact = od.paged_prefill(q[4:], kc, vc, tables, np.array([ctx]), np.array([0, 10]), 0.4,
                             "f32")
    assert not long[:4].any()
    assert np.array_equal(long[4:], exact)


def pin_prefill_gqa_is_repeated_mha(seed=26):
    rng = np.random.default_rng(seed)
    Hkv, G, D, bs = 2, 4, 8, 8
    lens, ns = [30, 17], [30, 9]
    Ks, Vs = contiguous_store(rng, lens, Hkv, D)
    kc, vc, tables = page_out(Ks, Vs, bs, 16, rng)
    q, qs = packed(rng, ns, Hkv * G, D)
    gqa = od.paged_prefill(q, kc, vc, tables, np.array(lens), qs, 0.3, "f32")
    kr, vr = np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1)
    mha = od.paged_prefill(q, kr, vr, tables, np.array(lens), qs, 0.3, "f32")
    assert np.array_equal(gqa, mha)


PINS = [pin_prefill_sdpa, pin_prefill_last_row_is_decode, pin_prefill_chunking,
        pin_prefill_closed_forms, pin_prefill_overlong_chunk, pin_prefill_gqa_is_repeated_mha]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
