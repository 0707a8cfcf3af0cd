"""Pins for the decode oracle (CPU only).

Each pin checks ``oracle.decode`` against something other than itself: the
hand-derived cases in ``tests/golden/decode_closed_form.json``, a dense masked
attention computed by ``torch.nn.functional.scaled_dot_product_attention`` in
float64 from a separately built contiguous store, closed forms, and
invariances that follow from the page-table reading of "PagedAttention: the KV
cache was the bottleneck all along", section "Virtual memory for attention"
(physical placement and block size do not change the result; forked sharing
equals copying).  ``test_oracle_mutants.py`` plants mistakes in the oracle and
checks that these pins catch each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.decode as od

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers: an independent contiguous store and its paged copy
# ---------------------------------------------------------------------------
def contiguous_store(rng, lens, Hkv, D):
    """Per-sequence contiguous K and V (float32 values), [ctx, Hkv, D] each."""
    return ([rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens],
            [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens])


def page_out(Ks, Vs, bs, NB, rng, MB=None):
    """Scatter contiguous sequences into a NaN-poisoned pool through random
    block tables; returns (k_cache, v_cache, tables)."""
    Hkv, D = Ks[0].shape[1:]
    need = [-(-len(k) // bs) for k in Ks]
    perm = rng.permutation(NB)
    mb = max(need) if MB is None else MB
    tables = np.full((len(Ks), mb), -1, dtype=np.int32)
    kc = np.full((NB, Hkv, bs, D), np.nan, dtype=np.float32)
    vc = np.full((NB, Hkv, bs, D), np.nan, dtype=np.float32)
    nxt = 0
    for s, (k, v) in enumerate(zip(Ks, Vs)):
        for j in range(need[s]):
            b = perm[nxt]
            nxt += 1
            tables[s, j] = b
            for i in range(bs):
                t = j * bs + i
                if t < len(k):
                    kc[b, :, i, :] = k[t]
                    vc[b, :, i, :] = v[t]
    return kc, vc, tables


def sdpa_reference(q, Ks, Vs, scale, Hq):
    """Dense masked attention from torch's library routine in float64."""
    S = len(Ks)
    Hkv, D = Ks[0].shape[1:]
    G = Hq // Hkv
    L = max(len(k) for k in Ks)
    Kd = torch.zeros(S, Hq, L, D, dtype=torch.float64)
    Vd = torch.zeros(S, Hq, L, D, dtype=torch.float64)
    mask = torch.zeros(S, 1, 1, L, dtype=torch.bool)
    for s in range(S):
        n = len(Ks[s])
        k = torch.from_numpy(Ks[s].astype(np.float64)).permute(1, 0, 2)   # [Hkv, n, D]
        v = torch.from_numpy(Vs[s].astype(np.float64)).permute(1, 0, 2)
        Kd[s, :, :n] = k.repeat_interleave(G, dim=0)
        Vd[s, :, :n] = v.repeat_interleave(G, dim=0)
        mask[s, ..., :n] = True
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kd, Vd, attn_mask=mask,
                                                         scale=float(np.float32(scale)))
    return o[:, :, 0, :].numpy()


def dense_numpy_reference(q, Ks, Vs, scale, Hq):
    """A second dense form: logits for all positions, -inf beyond ctx."""
    S = len(Ks)
    Hkv, D = Ks[0].shape[1:]
    G = Hq // Hkv
    L = max(len(k) for k in Ks)
    out = np.zeros((S, Hq, D))
    sc = float(np.float32(scale))
    for s in range(S):
        n = len(Ks[s])
        for h in range(Hq):
            logits = np.full(L, -np.inf)
            logits[:n] = sc * (Ks[s][:, h // G, :].astype(np.float64) @ q[s, h].astype(np.float64))
            w = np.exp(logits - logits.max())
            out[s, h] = (w[:n] / w.sum()) @ Vs[s][:, h // G, :].astype(np.float64)
    return out


def load_golden():
    with open(os.path.join(GOLDEN, "decode_closed_form.json")) as f:
        doc = json.load(f)
    cases = []
    for c in doc["cases"]:
        cases.append(dict(c, key_cache=np.array(_nan(c["key_cache"]), dtype=np.float32),
                          value_cache=np.array(_nan(c["value_cache"]), dtype=np.float32),
                          q=np.array(c["q"], dtype=np.float32),
                          block_tables=np.array(c["block_tables"], dtype=np.int32),
                          expected=np.array(c["expected"], dtype=np.float64)))
    return cases


def _nan(x):
    if isinstance(x, list):
        return [_nan(v) for v in x]
    return np.nan if x is None else x


# ---------------------------------------------------------------------------
# pins (plain functions so the mutant tests can run them against a broken oracle)
# ---------------------------------------------------------------------------
def pin_golden():
    for c in load_golden():
        got = od.paged_decode(c["q"], c["key_cache"], c["value_cache"], c["block_tables"],
                              c["context_lens"], c["scale"], "f32")
        assert got.shape == c["expected"].shape, c["name"]
        err = np.max(np.abs(got - c["expected"]))
        assert err <= c["atol"], (c["name"], err)


def pin_dense_library(seed=1):
    rng = np.random.default_rng(seed)
    for (S, Hq, Hkv, D, bs) in [(3, 4, 4, 8, 4), (4, 8, 2, 16, 8), (2, 6, 3, 4, 16)]:
        lens = rng.integers(1, 40, size=S)
        Ks, Vs = contiguous_store(rng, lens, Hkv, D)
        NB = int(sum(-(-n // bs) for n in lens)) + 5
        kc, vc, tab = page_out(Ks, Vs, bs, NB, rng)
        q = rng.standard_normal((S, Hq, D)).astype(np.float32)
        scale = 1.0 / math.sqrt(D)
        got = od.paged_decode(q, kc, vc, tab, lens, scale, "f32")
        ref = sdpa_reference(q, Ks, Vs, scale, Hq)
        ref2 = dense_numpy_reference(q, Ks, Vs, scale, Hq)
        assert np.max(np.abs(got - ref)) < 1e-12
        assert np.max(np.abs(got - ref2)) < 1e-12


def pin_physical_permutation(seed=2):
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, D, bs = 3, 4, 2, 8, 4
    lens = np.array([13, 1, 9])
    Ks, Vs = contiguous_store(rng, lens, Hkv, D)
    q = rng.standard_normal((S, Hq, D)).astype(np.float32)
    outs = []
    for trial in range(3):
        kc, vc, tab = page_out(Ks, Vs, bs, 20, np.random.default_rng(100 + trial))
        outs.append(od.paged_decode(q, kc, vc, tab, lens, 0.3, "f32"))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def pin_block_size(seed=3):
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, D = 3, 2, 2, 8
    lens = np.array([33, 7, 64])
    Ks, Vs = contiguous_store(rng, lens, Hkv, D)
    q = rng.standard_normal((S, Hq, D)).astype(np.float32)
    outs = []
    for bs in (1, 8, 16, 32):
        kc, vc, tab = page_out(Ks, Vs, bs, 200, rng)
        outs.append(od.paged_decode(q, kc, vc, tab, lens, 0.25, "f32"))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def pin_length_one(seed=4):
    rng = np.random.default_rng(seed)
    Ks, Vs = contiguous_store(rng, [1, 1], 2, 16)
    kc, vc, tab = page_out(Ks, Vs, 16, 4, rng)
    q = rng.standard_normal((2, 4, 16)).astype(np.float32)
    got = od.paged_decode(q, kc, vc, tab, [1, 1], 0.25, "f32")
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], Vs[s][0, h // 2].astype(np.float64))


def pin_fork_equals_copy(seed=5):
    """Two sequences sharing their first blocks (refcount 2) give the same
    output as the same tokens stored in private blocks."""
    rng = np.random.default_rng(seed)
    Hkv, D, bs = 2, 8, 4
    prefix_k = rng.standard_normal((10, Hkv, D)).astype(np.float32)
    prefix_v = rng.standard_normal((10, Hkv, D)).astype(np.float32)
    tails = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in (3, 6)]
    tails_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in (3, 6)]
    Ks = [np.concatenate([prefix_k[:8], t]) for t in tails]   # 8 = 2 full shared blocks
    Vs = [np.concatenate([prefix_v[:8], t]) for t in tails_v]
    q = rng.standard_normal((2, 2, D)).astype(np.float32)
    kc, vc, tab = page_out(Ks, Vs, bs, 12, rng)
    private = od.paged_decode(q, kc, vc, tab, [11, 14], 0.5, "f32")
    shared_tab = tab.copy()
    shared_tab[1, :2] = tab[0, :2]          # sequence 1 now reads sequence 0's prefix blocks
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[tab[1, :2]] = np.nan                # its own prefix copies are gone
    vc2[tab[1, :2]] = np.nan
    shared = od.paged_decode(q, kc2, vc2, shared_tab, [11, 14], 0.5, "f32")
    assert np.array_equal(private, shared)


def pin_closed_forms(seed=6):
    rng = np.random.default_rng(seed)
    Hkv, D, bs, n = 1, 8, 4, 11
    Vs = [rng.standard_normal((n, Hkv, D)).astype(np.float32)]
    mean = Vs[0][:, 0, :].astype(np.float64).mean(axis=0)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    # all keys equal -> uniform weights
    Ks = [np.repeat(rng.standard_normal((1, Hkv, D)).astype(np.float32), n, axis=0)]
    kc, vc, tab = page_out(Ks, Vs, bs, 5, rng)
    assert np.max(np.abs(od.paged_decode(q, kc, vc, tab, [n], 0.7, "f32")[0, 0] - mean)) < 1e-12
    # random keys, zero query or zero scale -> uniform weights
    Ks = [rng.standard_normal((n, Hkv, D)).astype(np.float32)]
    kc, vc, tab = page_out(Ks, Vs, bs, 5, rng)
    assert np.max(np.abs(od.paged_decode(np.zeros_like(q), kc, vc, tab, [n], 0.7, "f32")[0, 0]
                         - mean)) < 1e-12
    assert np.max(np.abs(od.paged_decode(q, kc, vc, tab, [n], 0.0, "f32")[0, 0] - mean)) < 1e-12
    # one dominant key: logit 40 above every other -> out = its value row within e^-Δ
    j = 6
    qv = q[0, 0].astype(np.float64)
    Ks = [np.zeros((n, Hkv, D), dtype=np.float32)]
    Ks[0][j, 0] = (40.0 * qv / (qv @ qv)).astype(np.float32)
    kc, vc, tab = page_out(Ks, Vs, bs, 5, rng)
    got = od.paged_decode(q, kc, vc, tab, [n], 1.0, "f32")[0, 0]
    assert np.max(np.abs(got - Vs[0][j, 0])) < n * math.exp(-39.0) * 10


def pin_gqa_is_repeated_mha(seed=7):
    rng = np.random.default_rng(seed)
    S, Hkv, G, D, bs = 2, 2, 4, 8, 8
    lens = [21, 5]
    Ks, Vs = contiguous_store(rng, lens, Hkv, D)
    q = rng.standard_normal((S, Hkv * G, D)).astype(np.float32)
    kc, vc, tab = page_out(Ks, Vs, bs, 8, rng)
    gqa = od.paged_decode(q, kc, vc, tab, lens, 0.35, "f32")
    mha = od.paged_decode(q, np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1), tab, lens,
                          0.35, "f32")
    assert np.array_equal(gqa, mha)


def pin_poison_only_where_no_token(seed=8):
    """NaN in unfilled tails and unused blocks never reaches the output, while
    NaN in a slot that holds an attended token does."""
    rng = np.random.default_rng(seed)
    Ks, Vs = contiguous_store(rng, [6, 9], 2, 4)
    kc, vc, tab = page_out(Ks, Vs, 4, 10, rng)
    q = rng.standard_normal((2, 2, 4)).astype(np.float32)
    assert np.isfinite(od.paged_decode(q, kc, vc, tab, [6, 9], 0.5, "f32")).all()
    vc[tab[1, 2], 1, 0, 0] = np.nan           # token 8 of sequence 1, head 1
    out = od.paged_decode(q, kc, vc, tab, [6, 9], 0.5, "f32")
    assert np.isfinite(out[0]).all() and np.isnan(out[1, 1, 0]) and np.isfinite(out[1, 0]).all()


def pin_widen():
    bf = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x7F80, 0x4049], dtype=np.uint16)
    w = od.widen(bf, "bf16")
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == 1.5
    assert w[3] == 2.0 ** -133 and np.isinf(w[4]) and w[5] == 3.140625
    h = np.array([1.0, -2.5, 65504.0, 2.0 ** -24], dtype=np.float16)
    assert list(od.widen(h, "f16")) == [1.0, -2.5, 65504.0, 2.0 ** -24]
    f = np.array([0.1], dtype=np.float32)
    assert od.widen(f, "f32")[0] == float(np.float32(0.1))


def pin_cache_write(seed=9):
    """A token written at the slot of logical position p is what the block
    table walk finds at p; every other byte is unchanged; slot -1 writes
    nothing."""
    rng = np.random.default_rng(seed)
    Hkv, D, bs, NB = 2, 4, 4, 6
    kc = rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32)
    vc = rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32)
    table = np.array([4, 1, 5], dtype=np.int32)
    positions = [0, 5, 10, 3]
    keys = rng.standard_normal((5, Hkv, D)).astype(np.float32)
    vals = rng.standard_normal((5, Hkv, D)).astype(np.float32)
    slots = [od.slot_of(table, p, bs) for p in positions] + [-1]
    assert slots[:4] == [16, 5, 22, 19]
    kc2, vc2 = od.reshape_and_cache(keys, vals, kc, vc, slots)
    K, V = od.gather_sequence(kc2, vc2, table, 11, bs, "f32")
    for t, p in enumerate(positions):
        assert np.array_equal(K[p], keys[t]) and np.array_equal(V[p], vals[t])
    touched = np.zeros((NB, bs), dtype=bool)
    for s in slots[:4]:
        touched[s // bs, s % bs] = True
    keep = ~touched[:, None, :, None].repeat(Hkv, 1).repeat(D, 3)
    assert np.array_equal(kc2[keep], kc[keep]) and np.array_equal(vc2[keep], vc[keep])
    assert not np.shares_memory(kc2, kc)


def pin_copy_blocks(seed=10):
    rng = np.random.default_rng(seed)
    layers = [rng.standard_normal((5, 2, 4, 3)).astype(np.float32) for _ in range(2)]
    vlayers = [rng.standard_normal((5, 2, 4, 3)).astype(np.float32) for _ in range(2)]
    ks, vs = od.copy_blocks(layers, vlayers, [(0, 3), (3, 4), (2, 0)])
    for L in range(2):
        k0, v0 = layers[L], vlayers[L]
        # applied in order: 3 <- 0, then 4 <- (new) 3 == old 0, then 0 <- 2
        assert np.array_equal(ks[L][3], k0[0]) and np.array_equal(ks[L][4], k0[0])
        assert np.array_equal(ks[L][0], k0[2]) and np.array_equal(vs[L][0], v0[2])
        assert np.array_equal(vs[L][4], v0[0])
        assert np.array_equal(ks[L][1], k0[1]) and np.array_equal(ks[L][2], k0[2])


def pin_byte_accounting():
    # A LLaMA-13B-shaped model (40 layers, 40 KV heads of 128, fp16) holding a
    # 2048-token sequence: the blog's "up to 1.7 GB" for one sequence
    # ("The number that made us read the code").
    per_tok = od.kv_bytes_per_token(40, 40, 128, 2)
    assert per_tok == 819200
    assert round(per_tok * 2048 / 1e9, 1) == 1.7
    assert od.algorithmic_kv_bytes([3, 5], 40, 128, 2) == 8 * 2 * 40 * 128 * 2


def pin_tail_waste():
    # Only the final block's tail is empty: fewer than bs slots per sequence.
    blocks, empty, frac = od.tail_waste([1, 16, 17, 33], 16)
    assert blocks == 1 + 1 + 2 + 3 and empty == 15 + 0 + 15 + 15
    assert frac == empty / (blocks * 16)


def pin_split_reduce_identity(seed=11):
    """Partitioned softmax recombined by max-rescaling equals the whole
    softmax (the algebra the split-context reduce relies on)."""
    rng = np.random.default_rng(seed)
    Ks, Vs = contiguous_store(rng, [100], 1, 8)
    kc, vc, tab = page_out(Ks, Vs, 16, 8, rng)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    whole = od.paged_decode(q, kc, vc, tab, [100], 0.9, "f32")[0, 0]
    K = Ks[0][:, 0].astype(np.float64)
    V = Vs[0][:, 0].astype(np.float64)
    z = float(np.float32(0.9)) * (K @ q[0, 0].astype(np.float64))
    for P in (1, 3, 7):
        parts = np.array_split(np.arange(100), P)
        m = np.array([z[i].max() for i in parts])
        l = np.array([np.exp(z[i] - mi).sum() for i, mi in zip(parts, m)])
        o = np.stack([np.exp(z[i] - mi) @ V[i] for i, mi in zip(parts, m)])
        M = m.max()
        w = np.exp(m - M)
        comb = (w[:, None] * o).sum(0) / (w * l).sum()
        assert np.max(np.abs(comb - whole)) < 1e-12


PINS = [pin_golden, pin_dense_library, pin_physical_permutation, pin_block_size,
        pin_length_one, pin_fork_equals_copy, pin_closed_forms, pin_gqa_is_repeated_mha,
        pin_poison_only_where_no_token, pin_widen, pin_cache_write, pin_copy_blocks,
        pin_byte_accounting, pin_tail_waste, pin_split_reduce_identity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
