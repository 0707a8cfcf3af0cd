"""Pins for the allocator oracle (CPU only).

Checked against the hand-traced run in ``tests/golden/allocator_trace.json``
and against invariants the pages fix for paged storage ("PagedAttention: the
KV cache was the bottleneck all along", section "Virtual memory for
attention"): blocks are acquired on demand so only the last block of an
unshared sequence is partly empty; shared blocks are copied only when a
sequence writes into one; forked and discarded sequences return their blocks.
"""
import copy
import json
import os

import numpy as np
import pytest

from oracle.alloc import Allocator, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def snapshot(a):
    return (list(a.ref), a.free_stack(), copy.deepcopy(a.tables), dict(a.lens))


def check_invariants(a):
    # every reference is one table entry or one registry entry; free +
    # referenced = pool
    counts = [0] * a.NB
    for t in a.tables.values():
        for b in t:
            counts[b] += 1
    for b in getattr(a, "registry", {}).values():
        counts[b] += 1
    assert counts == a.ref
    assert len(a.free) + sum(1 for r in a.ref if r > 0) == a.NB
    assert all(a.ref[b] == 0 for b in a.free)
    assert len(set(a.free)) == len(a.free)
    for sid, t in a.tables.items():
        assert len(t) == -(-a.lens[sid] // a.bs)       # ceil(len / bs) blocks


def pin_trace():
    with open(os.path.join(GOLDEN, "allocator_trace.json")) as f:
        doc = json.load(f)
    a = Allocator(doc["num_blocks"], doc["bs"])
    for op in doc["ops"]:
        kind = op["op"]
        if kind == "create":
            a.create(op["seq"])
        elif kind == "fork":
            before = a.num_free()
            a.fork(op["parent"], op["child"])
            assert a.num_free() == before
        elif kind == "release":
            a.release(op["seq"])
        elif kind == "append":
            if op["expect"] == "OOM":
                snap = snapshot(a)
                with pytest.raises(OutOfBlocks):
                    a.append(op["seq"])
                assert snapshot(a) == snap
            else:
                assert list(a.append(op["seq"])) == op["expect"], op["why"]
        check_invariants(a)
    fin = doc["final"]
    assert a.ref == fin["refcounts"]
    assert a.free_stack() == fin["free_stack"]
    assert {str(k): v for k, v in a.tables.items()} == fin["tables"]
    assert {str(k): v for k, v in a.lens.items()} == fin["lens"]


def pin_random_ops(seed=0, steps=3000):
    """Random create/append/fork/release with invariants after every step and
    an out-of-blocks attempt leaving the state untouched."""
    rng = np.random.default_rng(seed)
    a = Allocator(24, 4, init_order=rng.permutation(24))
    live, nxt = [], 0
    for _ in range(steps):
        r = rng.random()
        if r < 0.1 or not live:
            a.create(nxt)
            live.append(nxt)
            nxt += 1
        elif r < 0.75:
            sid = live[rng.integers(len(live))]
            snap = snapshot(a)
            before_len = a.seq_len(sid)
            shared_partial = (before_len % a.bs != 0 and a.ref[a.tables[sid][-1]] > 1)
            try:
                slot, src, dst = a.append(sid)
            except OutOfBlocks:
                assert snapshot(a) == snap
                assert a.num_free() == 0
                continue
            t = a.tables[sid]
            assert slot == t[-1] * a.bs + before_len % a.bs
            if shared_partial:
                assert src == snap[2][sid][-1] and dst == t[-1] and a.ref[dst] == 1
            else:
                assert (src, dst) == (-1, -1)
        elif r < 0.85:
            p = live[rng.integers(len(live))]
            free_before = a.num_free()
            a.fork(p, nxt)
            assert a.num_free() == free_before
            live.append(nxt)
            nxt += 1
        else:
            sid = live.pop(rng.integers(len(live)))
            a.release(sid)
        check_invariants(a)
    for sid in list(live):
        a.release(sid)
    assert a.num_free() == a.NB and all(r == 0 for r in a.ref)


def pin_tail_only_waste():
    a = Allocator(64, 16)
    for sid, n in enumerate([1, 16, 17, 100, 255]):
        a.create(sid)
        for _ in range(n):
            a.append(sid)
        blocks = a.tables[sid]
        assert len(blocks) * 16 - n < 16          # waste is below one block
        assert len(set(blocks)) == len(blocks)


def pin_tail_waste_closed_form():
    """The block-size cost model's waste term: blocks are acquired as a
    sequence grows, so only its last block has empty slots, bs - (n mod bs)
    of them unless n fills it.  Over one sequence per residue class the
    empty slots add up to exactly bs (bs - 1) / 2, i.e. (bs - 1) / 2 per
    sequence, the model's expected tail waste."""
    rng = np.random.default_rng(7)
    for bs in (8, 16, 32):
        a = Allocator(4096, bs)
        empty = 0
        for r in range(bs):
            n = bs * int(rng.integers(1, 4)) + r
            a.create(r)
            for _ in range(n):
                a.append(r)
            empty += len(a.tables[r]) * bs - n
        assert 2 * empty == bs * (bs - 1)


def pin_lazy_cow_count():
    """n sequences sharing a half-filled block: the first n-1 writers copy,
    the last one writes in place; a full shared block is never copied."""
    for prompt_len, expect in ((504, 3), (512, 0)):
        a = Allocator(64, 16)
        a.create(0)
        for _ in range(prompt_len):
            a.append(0)
        for c in (1, 2, 3):
            a.fork(0, c)
        pairs = [a.append(s)[1:] for s in range(4)]
        copies = [p for p in pairs if p != (-1, -1)]
        assert len(copies) == expect
        if expect:
            assert all(p[0] == a.tables[3][-1] for p in copies)
            assert a.ref[a.tables[3][-1]] == 1


def pin_sharing_saving():
    """Blocks held with sharing vs private copies for 4 samples of one
    512-token prompt with tails 0..3 blocks long."""
    a = Allocator(256, 16)
    a.create(0)
    for _ in range(512):
        a.append(0)
    for c in (1, 2, 3):
        a.fork(0, c)
    tails = [0, 16, 32, 48]
    for s, n in enumerate(tails):
        for _ in range(n):
            a.append(s)
    used = a.NB - a.num_free()
    private = sum(-(-(512 + n) // 16) for n in tails)
    assert used == 32 + 0 + 1 + 2 + 3
    assert private == 4 * 32 + 6
    assert abs((1 - used / private) - (1 - 38 / 134)) < 1e-15


def pin_prefix_trace():
    with open(os.path.join(GOLDEN, "prefix_registry_trace.json")) as f:
        doc = json.load(f)
    a = Allocator(doc["num_blocks"], doc["bs"])
    for op in doc["ops"]:
        kind, why = op["op"], op.get("why", op["op"])
        if kind == "create":
            a.create(op["seq"])
        elif kind == "append_n":
            assert [a.append(op["seq"])[0] for _ in range(op["n"])] == op["expect_slots"], why
        elif kind == "append":
            assert list(a.append(op["seq"])) == op["expect"], why
        elif kind == "publish":
            assert a.publish(op["seq"], op["keys"]) == op["expect"], why
        elif kind == "create_prefixed":
            assert a.create_prefixed(op["seq"], op["keys"]) == op["expect"], why
            assert a.table(op["seq"]) == op["table"] and a.seq_len(op["seq"]) == op["len"], why
        elif kind == "evict":
            assert a.evict(op["keys"]) == op["expect"], why
        elif kind == "release":
            a.release(op["seq"])
        assert a.ref == op["ref_after"], why
        assert a.free_stack() == op["free_after"], why
        check_invariants(a)
    assert len(a.registry) == doc["final_registry_size"] and not a.tables


def pin_prefix_random_ops(seed=1, steps=3000):
    """Random requests that publish and reuse chained prefixes, forks,
    appends, releases and evictions, with the invariants after every step:
    references = table entries + registry entries, registered blocks are never
    free, a prefixed sequence starts with registered blocks, and appending
    after a full match never copies."""
    rng = np.random.default_rng(seed)
    a = Allocator(48, 4, init_order=rng.permutation(48))
    # chained keys of four "system prompts" of 1..6 blocks
    prompts = [[1000 * p + j for j in range(int(rng.integers(1, 7)))] for p in range(4)]
    live, nxt = [], 0
    for _ in range(steps):
        r = rng.random()
        try:
            if r < 0.12 or not live:
                keys = prompts[rng.integers(4)]
                n = int(rng.integers(0, len(keys) + 1))
                m = a.create_prefixed(nxt, keys[:n])
                assert a.table(nxt) == [a.registry[k] for k in keys[:m]]
                assert m == n or keys[m] not in a.registry
                assert a.seq_len(nxt) == m * a.bs
                live.append(nxt)
                nxt += 1
                if m:
                    slot, src, dst = a.append(nxt - 1)       # full blocks: no copy
                    assert (src, dst) == (-1, -1)
            elif r < 0.6:
                sid = live[rng.integers(len(live))]
                a.append(sid)
            elif r < 0.7:
                sid = live[rng.integers(len(live))]
                keys = prompts[rng.integers(4)]
                n = min(len(keys), a.seq_len(sid) // a.bs)
                before = dict(a.registry)
                added = a.publish(sid, keys[:n])
                assert added == sum(1 for k in keys[:n] if k not in before)
                assert all(a.registry[k] == before[k] for k in before)
            elif r < 0.78:
                p = live[rng.integers(len(live))]
                a.fork(p, nxt)
                live.append(nxt)
                nxt += 1
            elif r < 0.88:
                a.release(live.pop(rng.integers(len(live))))
            else:
                keys = prompts[rng.integers(4)]
                present = sum(1 for k in keys if k in a.registry)
                assert a.evict(keys) == present
        except OutOfBlocks:
            pass
        check_invariants(a)
        assert not set(a.registry.values()) & set(a.free)
    for sid in list(live):
        a.release(sid)
    for keys in prompts:
        a.evict(keys)
    assert a.num_free() == a.NB and all(r == 0 for r in a.ref) and not a.registry


def pin_system_prompt_saving():
    """N requests that share a 64-block system prompt through the registry
    hold 64 + their own blocks; private prompts would hold N * 64 more."""
    a = Allocator(1024, 16)
    keys = list(range(64))
    a.create(0)
    for _ in range(64 * 16):
        a.append(0)
    assert a.publish(0, keys) == 64
    own = [0, 1, 15, 16, 17, 100]
    for r, n in enumerate(own, start=1):
        assert a.create_prefixed(r, keys) == 64
        for _ in range(n):
            assert a.append(r)[1:] == (-1, -1)
    used = a.NB - a.num_free()
    mine = sum(-(-n // 16) for n in own)
    assert used == 64 + mine
    private = (len(own) + 1) * 64 + mine
    assert private - used == len(own) * 64


PINS = [pin_trace, pin_random_ops, pin_tail_only_waste, pin_tail_waste_closed_form, pin_lazy_cow_count, pin_sharing_saving,
        pin_prefix_trace, pin_prefix_random_ops, pin_system_prompt_saving]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
