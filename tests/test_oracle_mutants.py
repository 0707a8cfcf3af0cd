"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant below is a plausible slip in ``oracle.decode`` or
``oracle.alloc`` (a dropped term, a wrong sign or index, a swapped operand, a
wrong tie-break).  The test swaps it into the oracle module for the duration
of one check and asserts that at least one pin fails; this is what makes the
pins worth trusting.
"""
import numpy as np
import pytest

import oracle.alloc as oa
import oracle.decode as od
import test_oracle_alloc as alloc_pins
import test_oracle_pins as decode_pins
import test_oracle_prefill_pins as prefill_pins


# ---- decode mutants -------------------------------------------------------
def attend_no_scale(qh, K, V, scale):
    z = K @ qh
    p = np.exp(z - z.max())
    return (p @ V) / p.sum()


def attend_wrong_sign(qh, K, V, scale):
    z = scale * (K @ qh)
    p = np.exp(z.min() - z)
    return (p @ V) / p.sum()


def attend_mean_denominator(qh, K, V, scale):
    z = scale * (K @ qh)
    p = np.exp(z - z.max())
    return (p @ V) / len(p)


def attend_keys_as_values(qh, K, V, scale):
    z = scale * (K @ qh)
    p = np.exp(z - z.max())
    return (p @ K) / p.sum()


def attend_drops_last_token(qh, K, V, scale):
    z = scale * (K[:-1] @ qh) if len(K) > 1 else scale * (K @ qh)
    Vv = V[:-1] if len(K) > 1 else V
    p = np.exp(z - z.max())
    return (p @ Vv) / p.sum()


def gather_swapped_index(k_cache, v_cache, table_row, ctx, bs, kv_dtype):
    need = -(-ctx // bs)
    blocks = np.asarray(table_row[:need], dtype=np.int64)
    pos = np.arange(ctx)
    phys = blocks[np.minimum(pos % bs, need - 1)]
    off = np.minimum(pos // bs, bs - 1)
    return (od.widen(k_cache[phys, :, off, :], kv_dtype),
            od.widen(v_cache[phys, :, off, :], kv_dtype))


def gather_ignores_table(k_cache, v_cache, table_row, ctx, bs, kv_dtype):
    pos = np.arange(ctx)
    phys = pos // bs
    return (od.widen(k_cache[phys, :, pos % bs, :], kv_dtype),
            od.widen(v_cache[phys, :, pos % bs, :], kv_dtype))


def widen_bf16_wrong_shift(a, kv_dtype):
    if kv_dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(8)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def slot_of_swapped(table_row, pos, bs):
    return int(table_row[pos % bs]) * bs + pos // bs


def reshape_and_cache_swapped(key, value, k_cache, v_cache, slot_mapping, inplace=False):
    kc, vc = k_cache.copy(), v_cache.copy()
    bs = kc.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        off, b = divmod(int(slot), bs)
        if b < kc.shape[0] and off < bs:
            kc[b, :, off, :] = key[t]
            vc[b, :, off, :] = value[t]
    return kc, vc


def copy_blocks_reversed(k_caches, v_caches, block_mapping, inplace=False):
    kcs = [k.copy() for k in k_caches]
    vcs = [v.copy() for v in v_caches]
    for src, dst in np.asarray(block_mapping).reshape(-1, 2).tolist():
        for kc, vc in zip(kcs, vcs):
            kc[src] = kc[dst]
            vc[src] = vc[dst]
    return kcs, vcs


def copy_blocks_keys_only(k_caches, v_caches, block_mapping, inplace=False):
    kcs = [k.copy() for k in k_caches]
    vcs = [v.copy() for v in v_caches]
    for src, dst in np.asarray(block_mapping).reshape(-1, 2).tolist():
        for kc in kcs:
            kc[dst] = kc[src]
    return kcs, vcs


def bytes_per_token_no_values(layers, Hkv, D, elem_bytes):
    return layers * Hkv * D * elem_bytes


def paged_decode_modulo_heads(q, k_cache, v_cache, block_tables, context_lens, scale,
                              kv_dtype, seqs=None):
    S, Hq, D = q.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    sc = float(np.float32(scale))
    out = np.empty((S, Hq, D))
    for s in range(S):
        K, V = od.gather_sequence(k_cache, v_cache, block_tables[s], int(context_lens[s]), bs,
                                  kv_dtype)
        qs = od.widen(q[s], kv_dtype)
        for h in range(Hq):
            out[s, h] = od.attend(qs[h], K[:, h % Hkv, :], V[:, h % Hkv, :], sc)
    return out


DECODE_MUTANTS = {
    "no_scale": ("attend", attend_no_scale),
    "wrong_sign": ("attend", attend_wrong_sign),
    "mean_denominator": ("attend", attend_mean_denominator),
    "keys_as_values": ("attend", attend_keys_as_values),
    "drops_last_token": ("attend", attend_drops_last_token),
    "gather_swapped_index": ("gather_sequence", gather_swapped_index),
    "gather_ignores_table": ("gather_sequence", gather_ignores_table),
    "widen_bf16_shift": ("widen", widen_bf16_wrong_shift),
    "slot_swapped": ("slot_of", slot_of_swapped),
    "cache_write_swapped": ("reshape_and_cache", reshape_and_cache_swapped),
    "copy_reversed": ("copy_blocks", copy_blocks_reversed),
    "copy_keys_only": ("copy_blocks", copy_blocks_keys_only),
    "bytes_no_values": ("kv_bytes_per_token", bytes_per_token_no_values),
    "modulo_heads": ("paged_decode", paged_decode_modulo_heads),
}


def caught(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name, monkeypatch):
    attr, fn = DECODE_MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    assert caught(decode_pins.PINS) is not None, f"mutant {name} passed every pin"


# ---- prefill mutants ------------------------------------------------------
def _prefill_with(rule):
    """A prefill oracle whose row i of a chunk attends the key prefix
    rule(i, n, ctx) -> end (exclusive), with heads mapped by ``head``."""
    def fn(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, kv_dtype,
           seqs=None, head=lambda h, G, Hkv: h // G, rows=lambda i, n: i):
        T, Hq, D = q.shape
        Hkv, bs = k_cache.shape[1], k_cache.shape[2]
        G = Hq // Hkv
        out = np.zeros((T, Hq, D))
        for s in range(len(context_lens)):
            r0, r1 = int(query_start[s]), int(query_start[s + 1])
            n, ctx = r1 - r0, int(context_lens[s])
            if n <= 0 or ctx <= 0:
                continue
            K, V = od.gather_sequence(k_cache, v_cache, block_tables[s], ctx, bs, kv_dtype)
            qs = od.widen(q[r0:r1], kv_dtype)
            for i in range(n):
                end = rule(i, n, ctx)
                if end <= 0:
                    continue
                for h in range(Hq):
                    g = head(h, G, Hkv)
                    out[r0 + i, h] = od.attend(qs[rows(i, n), h], K[:end, g], V[:end, g],
                                               float(np.float32(scale)))
        return out
    return fn


def _with(rule, **kw):
    base = _prefill_with(rule)
    return lambda *a, **k: base(*a, **{**k, **kw})


PREFILL_MUTANTS = {
    "causal_excludes_self": _prefill_with(lambda i, n, ctx: ctx - n + i),
    "position_from_chunk_start": _prefill_with(lambda i, n, ctx: i + 1),
    "not_causal": _prefill_with(lambda i, n, ctx: ctx),
    "modulo_heads": _with(lambda i, n, ctx: ctx - n + i + 1, head=lambda h, G, Hkv: h % Hkv),
    "rows_reversed": _with(lambda i, n, ctx: ctx - n + i + 1, rows=lambda i, n: n - 1 - i),
}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(od, "paged_prefill", PREFILL_MUTANTS[name])
    assert caught(prefill_pins.PINS) is not None, f"mutant {name} passed every pin"


def test_prefill_reference_rule_passes(monkeypatch):
    # the harness itself: the correct rule written the same way passes
    monkeypatch.setattr(od, "paged_prefill", _prefill_with(lambda i, n, ctx: ctx - n + i + 1))
    assert caught(prefill_pins.PINS) is None


# ---- allocator mutants ----------------------------------------------------
class FifoAllocator(oa.Allocator):
    def _pop(self):
        b = self.free.pop(0)
        self.ref[b] = 1
        return b


class EagerCowAllocator(oa.Allocator):
    """Copies a partly filled last block at fork time instead of on write."""
    def fork(self, parent, child):
        super().fork(parent, child)
        if self.lens[child] % self.bs and self.free:
            last = self.tables[child][-1]
            self.ref[last] -= 1
            self.tables[child][-1] = self._pop()


class ForwardReleaseAllocator(oa.Allocator):
    def release(self, sid):
        table = self.tables.pop(sid)
        del self.lens[sid]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)


class NoCowAllocator(oa.Allocator):
    def append(self, sid):
        n = self.lens[sid]
        if n % self.bs == 0:
            if not self.free:
                raise oa.OutOfBlocks()
            self.tables[sid].append(self._pop())
        self.lens[sid] = n + 1
        return self.tables[sid][-1] * self.bs + n % self.bs, -1, -1


class LeakyReleaseAllocator(oa.Allocator):
    def release(self, sid):
        table = self.tables.pop(sid)
        del self.lens[sid]
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0 and b != table[0]:
                self.free.append(b)


class PublishNoRefAllocator(oa.Allocator):
    """The registry does not hold a reference to its blocks."""
    def publish(self, sid, keys):
        added = 0
        for j, k in enumerate(int(k) for k in keys):
            if k not in self.registry:
                self.registry[k] = self.tables[sid][j]
                added += 1
        return added


class PublishOverwriteAllocator(oa.Allocator):
    """A repeated key takes the newer block (last publisher wins)."""
    def publish(self, sid, keys):
        added = 0
        for j, k in enumerate(int(k) for k in keys):
            b = self.tables[sid][j]
            if k in self.registry:
                old = self.registry[k]
                if old == b:
                    continue
                self.ref[old] -= 1
                if self.ref[old] == 0:
                    self.free.append(old)
            else:
                added += 1
            self.registry[k] = b
            self.ref[b] += 1
        return added


class PrefixSkipsMissAllocator(oa.Allocator):
    """Takes every present key instead of stopping at the first miss."""
    def create_prefixed(self, sid, keys):
        blocks = [self.registry[int(k)] for k in keys if int(k) in self.registry]
        for b in blocks:
            self.ref[b] += 1
        self.tables[sid] = blocks
        self.lens[sid] = len(blocks) * self.bs
        return len(blocks)


class PrefixZeroLengthAllocator(oa.Allocator):
    """Shares the blocks but forgets the tokens they hold."""
    def create_prefixed(self, sid, keys):
        m = super().create_prefixed(sid, keys)
        self.lens[sid] = 0
        return m


class ForwardEvictAllocator(oa.Allocator):
    def evict(self, keys):
        removed = 0
        for k in (int(k) for k in keys):
            if k in self.registry:
                b = self.registry.pop(k)
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self.free.append(b)
                removed += 1
        return removed


ALLOC_MUTANTS = {"fifo": FifoAllocator, "eager_cow": EagerCowAllocator,
                 "forward_release": ForwardReleaseAllocator, "no_cow": NoCowAllocator,
                 "leaky_release": LeakyReleaseAllocator, "publish_no_ref": PublishNoRefAllocator,
                 "publish_overwrite": PublishOverwriteAllocator,
                 "prefix_skips_miss": PrefixSkipsMissAllocator,
                 "prefix_zero_length": PrefixZeroLengthAllocator,
                 "forward_evict": ForwardEvictAllocator}


@pytest.mark.parametrize("name", sorted(ALLOC_MUTANTS))
def test_alloc_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(alloc_pins, "Allocator", ALLOC_MUTANTS[name])
    assert caught(alloc_pins.PINS) is not None, f"mutant {name} passed every pin"
