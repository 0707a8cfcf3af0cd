"""Oracle: paged single-query decode attention, cache write and block copy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): float64 numpy, no
blocking or fusion beyond what the definitions say.

Storage conventions shared with the inputs (not with the GPU code):
  * a KV pool is ``[NB, Hkv, bs, D]``: block ``b`` holds, for every KV head,
    ``bs`` consecutive token rows of ``D`` elements;
  * float32 / float16 arrays hold themselves, bfloat16 arrays hold uint16 bit
    patterns (numpy has no bfloat16);
  * a block table row lists physical block numbers in logical order; entries
    past ``ceil(ctx / bs)`` are never read.
"""
from __future__ import annotations

import numpy as np


def widen(a: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored KV/query elements -> float64, exactly.

    bfloat16 is the upper half of a float32: shifting its 16 bits left by 16
    gives that float32, which float64 represents exactly.
    """
    if kv_dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if kv_dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def slot_of(table_row: np.ndarray, pos: int, bs: int) -> int:
    """Physical slot of logical token ``pos``: the block table maps the
    logical block ``pos // bs`` to a physical block, as a page table maps a
    virtual page to a frame, and the offset inside the block is kept
    ("PagedAttention: the KV cache was the bottleneck all along", section
    "Virtual memory for attention")."""
    return int(table_row[pos // bs]) * bs + pos % bs


def gather_sequence(k_cache, v_cache, table_row, ctx: int, bs: int, kv_dtype: str):
    """Materialise one sequence's contiguous keys and values, float64
    ``[ctx, Hkv, D]`` each, by walking its block table token by token
    ("Virtual memory for attention": keys and values are gathered from blocks
    that need not be adjacent)."""
    NB = k_cache.shape[0]
    need = -(-ctx // bs)
    blocks = np.asarray(table_row[:need], dtype=np.int64)
    if np.any(blocks < 0) or np.any(blocks >= NB):
        raise ValueError("block table entry outside the pool")
    pos = np.arange(ctx)
    phys = blocks[pos // bs]
    off = pos % bs
    K = widen(k_cache[phys, :, off, :], kv_dtype)
    V = widen(v_cache[phys, :, off, :], kv_dtype)
    return K, V


def attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook single-query attention in float64:
    ``softmax(scale * K @ q) @ V`` with the maximum logit subtracted first
    (identical in exact arithmetic; it keeps exp() in range)."""
    z = scale * (K @ qh)
    p = np.exp(z - z.max())
    return (p @ V) / p.sum()


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                 kv_dtype: str, seqs=None) -> np.ndarray:
    """Decode attention for one new query token per sequence.

    ``q`` is ``[S, Hq, D]`` in the KV dtype's storage; ``context_lens[s]``
    counts the tokens attended, the step's own token included.  Query head
    ``h`` reads KV head ``h // (Hq // Hkv)`` (consecutive query heads share a
    KV head; with ``Hq == Hkv`` this is plain multi-head attention).  The
    scale is the float32 value the GPU receives, widened.

    Returns float64 ``[len(seqs), Hq, D]`` (all sequences by default).
    """
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    bs = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    sc = float(np.float32(scale))
    seqs = range(S) if seqs is None else seqs
    out = []
    for s in seqs:
        ctx = int(context_lens[s])
        if ctx < 1:
            raise ValueError("context length must be >= 1")
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], ctx, bs, kv_dtype)
        qs = widen(q[s], kv_dtype)
        o = np.empty((Hq, D), dtype=np.float64)
        for h in range(Hq):
            g = h // G
            o[h] = attend(qs[h], K[:, g, :], V[:, g, :], sc)
        out.append(o)
    return np.stack(out) if out else np.zeros((0, Hq, D))


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                  kv_dtype: str, seqs=None) -> np.ndarray:
    """Causal attention for a chunk of new tokens per sequence (prefill).

    The pages fix only where the keys live ("PagedAttention: the KV cache was
    the bottleneck all along", section "Virtual memory for attention": a
    prompt's tokens go into blocks acquired as the sequence grows, and
    attention gathers them through the block table).  Reading taken: the
    chunk of sequence ``s`` is the last ``n = query_start[s+1] -
    query_start[s]`` of its ``ctx = context_lens[s]`` tokens, already in the
    pool; its token ``i`` sits at position ``p = ctx - n + i`` and attends to
    positions ``0 .. p`` (itself included), the usual causal rule of a
    decoder.  Rows whose position would be negative (``n > ctx``) are zero.

    ``q`` is ``[T, Hq, D]`` (rows ``query_start[s] ..`` belong to ``s``), in
    the KV dtype's storage.  Returns float64 ``[T, Hq, D]``; rows of
    sequences not in ``seqs`` (all by default) are left zero.
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    bs = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    sc = float(np.float32(scale))
    S = len(context_lens)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        n, ctx = r1 - r0, int(context_lens[s])
        if n <= 0 or ctx <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], ctx, bs, kv_dtype)
        qs = widen(q[r0:r1], kv_dtype)
        for i in range(n):
            p = ctx - n + i
            if p < 0:
                continue
            for h in range(Hq):
                g = h // G
                out[r0 + i, h] = attend(qs[i, h], K[:p + 1, g, :], V[:p + 1, g, :], sc)
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, inplace=False):
    """Cache write: token ``t``'s K and V rows (``[T, Hkv, D]``) go to physical
    slot ``slot_mapping[t]`` of the pools, i.e. block ``slot // bs`` at offset
    ``slot % bs`` for every head; a slot of -1 means "no write".  All other
    bytes are unchanged.  Returns the (possibly copied) pools."""
    kc = k_cache if inplace else k_cache.copy()
    vc = v_cache if inplace else v_cache.copy()
    bs = kc.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, off = divmod(int(slot), bs)
        kc[b, :, off, :] = key[t]
        vc[b, :, off, :] = value[t]
    return kc, vc


def copy_blocks(k_caches, v_caches, block_mapping, inplace=False):
    """Copy-on-write block copy: for each ``(src, dst)`` pair, in list order,
    every layer's K block and V block ``dst`` become copies of block ``src``
    (one block number names both the keys and the values it holds).  Pairs are
    applied one after another."""
    kcs = [k if inplace else k.copy() for k in k_caches]
    vcs = [v if inplace else v.copy() for v in v_caches]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2).tolist():
        for kc, vc in zip(kcs, vcs):
            kc[dst] = kc[src]
            vc[dst] = vc[src]
    return kcs, vcs


def kv_bytes_per_token(layers: int, Hkv: int, D: int, elem_bytes: int) -> int:
    """KV cache bytes one token occupies: a key and a value row per KV head
    per layer."""
    return 2 * layers * Hkv * D * elem_bytes


def algorithmic_kv_bytes(context_lens, Hkv: int, D: int, elem_bytes: int) -> int:
    """Bytes a decode step must read: every attended token's K and V rows once
    per KV head (one layer)."""
    return int(np.sum(np.asarray(context_lens, dtype=np.int64))) * kv_bytes_per_token(
        1, Hkv, D, elem_bytes)


def tail_waste(context_lens, bs: int):
    """Unshared paged storage: blocks used, token slots left empty, and the
    empty fraction.  Only the last block of a sequence can be partly empty
    ("Virtual memory for attention")."""
    lens = np.asarray(context_lens, dtype=np.int64)
    blocks = -(-lens // bs)
    empty = int(np.sum(blocks * bs - lens))
    total = int(np.sum(blocks)) * bs
    return int(np.sum(blocks)), empty, (empty / total if total else 0.0)
