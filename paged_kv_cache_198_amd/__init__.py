"""Paged KV cache decode path for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libpa.so`` (C ABI in ``include/pa.h``).  The
functions below only check and marshal arguments (torch tensors -> device
pointers and sizes, the current torch stream -> hipStream_t); every step of
the computation runs in the library's HIP kernels or its C++ allocator.  There
is no fallback: if ``libpa.so`` is missing, every call raises.

Names follow the C ABI: ``pa_reshape_and_cache``, ``pa_decode_attention``,
``pa_decode_step`` (the two fused), ``pa_decode_workspace_bytes``,
``pa_copy_blocks``, ``pa_cascade_plan`` / ``pa_decode_cascade`` (shared-prefix
decode), ``pa_prefill_attention`` (causal attention over a chunk of new
tokens); ``Allocator`` wraps the ``pa_alloc_*`` / ``pa_seq_*``
calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # loads the HIP runtime libpa.so then binds to (one runtime per process)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
_DTYPE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
_ELEM = {PA_F32: 4, PA_F16: 2, PA_BF16: 2}

PA_OK, PA_ERR_INVALID, PA_ERR_OOM, PA_ERR_HIP, PA_ERR_WORKSPACE, PA_ERR_UNSUPPORTED = (
    0, -1, -2, -3, -4, -5)
PA_ERR_TOO_LARGE = -6
PA_STATIC_SCRATCH_BYTES = 32 << 20   # the no-alloc step's static workspace per GPU

_lib = None

_c_int, _c_i32, _c_i64, _c_p = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_p_i32 = ctypes.POINTER(ctypes.c_int32)
_p_i64 = ctypes.POINTER(ctypes.c_int64)
_p_u64 = ctypes.POINTER(ctypes.c_uint64)

_SIGNATURES = {
    "pa_version": (_c_int, []),
    "pa_status_string": (ctypes.c_char_p, [_c_int]),
    "pa_reshape_and_cache": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _c_i32, _c_p]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_attention": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                     _c_i32, _c_p, ctypes.c_size_t, _c_i32, _c_p]),
    "pa_decode_step": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_float,
                                _c_i32, _c_p, ctypes.c_size_t, _c_i32, _c_p]),
    "pa_decode_step_noalloc": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        ctypes.c_float, _c_i32, _c_i32, _c_p]),
    "pa_cascade_plan": (_c_int, [_p_i32, _p_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                 _c_i32, _p_i32, ctypes.c_size_t, _p_i32]),
    "pa_cascade_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_cascade": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                   _c_i32, ctypes.c_float, _c_i32, _c_p, ctypes.c_size_t, _c_i32,
                                   _c_p]),
    "pa_prefill_attention": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                      ctypes.c_float, _c_i32, _c_p]),
    "pa_probe_read_bandwidth": (_c_int, [_c_p, ctypes.c_size_t, _c_p, _c_i32, _c_p]),
    "pa_copy_blocks": (_c_int, [ctypes.POINTER(_c_p), ctypes.POINTER(_c_p), _c_i32, _p_i64,
                                _c_i32, _c_i32, _c_i64, _c_p]),
    "pa_alloc_create": (_c_p, [_c_i32, _c_i32, _p_i32]),
    "pa_alloc_destroy": (None, [_c_p]),
    "pa_alloc_num_free": (_c_i32, [_c_p]),
    "pa_alloc_num_blocks": (_c_i32, [_c_p]),
    "pa_alloc_block_size": (_c_i32, [_c_p]),
    "pa_alloc_refcount": (_c_i32, [_c_p, _c_i32]),
    "pa_seq_create": (_c_int, [_c_p, _c_i64]),
    "pa_seq_append": (_c_int, [_c_p, _c_i64, _p_i64, _p_i64, _p_i64]),
    "pa_seq_append_n": (_c_int, [_c_p, _c_i64, _c_i32, _p_i64, _p_i64, _p_i64]),
    "pa_seq_fork": (_c_int, [_c_p, _c_i64, _c_i64]),
    "pa_seq_free": (_c_int, [_c_p, _c_i64]),
    "pa_seq_len": (_c_i32, [_c_p, _c_i64]),
    "pa_seq_num_blocks": (_c_i32, [_c_p, _c_i64]),
    "pa_seq_blocks": (_c_int, [_c_p, _c_i64, _p_i32, _c_i32]),
    "pa_build_batch": (_c_int, [_c_p, _p_i64, _c_i32, _c_i32, _p_i32, _p_i32]),
    "pa_alloc_export": (_c_int, [_c_p, _p_i32, _p_i32, _p_i32]),
    "pa_prefix_publish": (_c_int, [_c_p, _c_i64, _p_u64, _c_i32, _p_i32]),
    "pa_seq_create_prefixed": (_c_int, [_c_p, _c_i64, _p_u64, _c_i32, _p_i32]),
    "pa_prefix_evict": (_c_int, [_c_p, _p_u64, _c_i32, _p_i32]),
    "pa_prefix_size": (_c_i32, [_c_p]),
}
EXPORTED = tuple(_SIGNATURES)


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class OutOfBlocks(PaError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_198_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(rc: int, where: str) -> None:
    if rc == PA_ERR_OOM:
        raise OutOfBlocks(rc, where)
    if rc != PA_OK:
        raise PaError(rc, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise ValueError(f"unsupported KV dtype {t.dtype}")
    return _DTYPE[t.dtype]


# ---------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------
def pa_reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                         stream=None) -> None:
    """Write each token's key/value rows ([T, Hkv, D]) into its slot of the
    [NB, Hkv, bs, D] pools; slot -1 = no write."""
    dt = _kv_dtype(key_cache)
    NB, Hkv, bs, D = key_cache.shape
    T = key.shape[0]
    for name, t in (("key", key), ("value", value)):
        if tuple(t.shape) != (T, Hkv, D) or t.dtype != key_cache.dtype:
            raise ValueError(f"{name} must be [T, {Hkv}, {D}] {key_cache.dtype}")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be [T]")
    rc = lib().pa_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping", torch.int64),
        T, Hkv, D, bs, NB, dt, _stream(stream))
    _check(rc, "pa_reshape_and_cache")


def pa_decode_workspace_bytes(S: int, Hq: int, D: int, max_context_len: int,
                              partition_tokens: int) -> int:
    return int(lib().pa_decode_workspace_bytes(S, Hq, D, max_context_len, partition_tokens))


def pa_decode_attention(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                        value_cache: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, max_context_len: int, scale: float,
                        partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """Paged single-query decode attention; ``out`` and ``query`` are
    [S, Hq, D] in the pools' dtype."""
    dt = _kv_dtype(key_cache)
    NB, Hkv, bs, D = key_cache.shape
    S, Hq, Dq = query.shape
    if Dq != D or query.dtype != key_cache.dtype:
        raise ValueError("query must be [S, Hq, D] in the KV dtype")
    if tuple(out.shape) != (S, Hq, D) or out.dtype != key_cache.dtype:
        raise ValueError("out must be [S, Hq, D] in the KV dtype")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, MB]")
    if tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be [S]")
    MB = block_tables.shape[1]
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().pa_decode_attention(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), float(scale), int(partition_tokens), ws_ptr, ws_bytes, dt,
        _stream(stream))
    _check(rc, "pa_decode_attention")


def _step_shapes(out, query, key, value, key_cache, value_cache, block_tables, context_lens):
    """Checks the fused step's tensors; (dtype code, S, Hq, Hkv, D, bs, NB, MB)."""
    dt = _kv_dtype(key_cache)
    NB, Hkv, bs, D = key_cache.shape
    S, Hq, Dq = query.shape
    if Dq != D or query.dtype != key_cache.dtype:
        raise ValueError("query must be [S, Hq, D] in the KV dtype")
    if tuple(out.shape) != (S, Hq, D) or out.dtype != key_cache.dtype:
        raise ValueError("out must be [S, Hq, D] in the KV dtype")
    for name, t in (("key", key), ("value", value)):
        if tuple(t.shape) != (S, Hkv, D) or t.dtype != key_cache.dtype:
            raise ValueError(f"{name} must be [S, {Hkv}, {D}] {key_cache.dtype}")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, MB]")
    if tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be [S]")
    return dt, S, Hq, Hkv, D, bs, NB, block_tables.shape[1]


def pa_decode_step(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                   key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, max_context_len: int, scale: float,
                   partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Fused step: store key[s]/value[s] ([S, Hkv, D]) at position
    context_lens[s]-1 of each sequence and attend over its whole context."""
    dt, S, Hq, Hkv, D, bs, NB, MB = _step_shapes(out, query, key, value, key_cache, value_cache,
                                                 block_tables, context_lens)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().pa_decode_step(
        _dev(out, "out"), _dev(query, "query"), _dev(key, "key"), _dev(value, "value"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), float(scale), int(partition_tokens), ws_ptr, ws_bytes, dt,
        _stream(stream))
    _check(rc, "pa_decode_step")


def pa_decode_step_noalloc(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor,
                           value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float, partition_tokens: int = 0,
                           stream=None) -> None:
    """The fused step with no workspace argument: partials go to the
    library's static per-GPU scratch (PA_STATIC_SCRATCH_BYTES); raises
    PaError(PA_ERR_TOO_LARGE) when the launch would need more."""
    dt, S, Hq, Hkv, D, bs, NB, MB = _step_shapes(out, query, key, value, key_cache, value_cache,
                                                 block_tables, context_lens)
    rc = lib().pa_decode_step_noalloc(
        _dev(out, "out"), _dev(query, "query"), _dev(key, "key"), _dev(value, "value"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), float(scale), int(partition_tokens), dt, _stream(stream))
    _check(rc, "pa_decode_step_noalloc")


def make_workspace(S: int, Hq: int, D: int, max_context_len: int, partition_tokens: int,
                   device="cuda") -> Optional[torch.Tensor]:
    """A workspace tensor of the required size (None when none is needed)."""
    n = pa_decode_workspace_bytes(S, Hq, D, max_context_len, partition_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def pa_prefill_attention(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, query_start: torch.Tensor,
                         max_query_len: int, scale: float, stream=None) -> None:
    """Causal attention for each sequence's chunk of new tokens: ``query`` and
    ``out`` are [T, Hq, D], sequence s owning rows query_start[s] ..
    query_start[s+1] ([S+1] int32), whose keys are the last rows of its
    context_lens[s] tokens in the pools."""
    dt = _kv_dtype(key_cache)
    NB, Hkv, bs, D = key_cache.shape
    T, Hq, Dq = query.shape
    if Dq != D or query.dtype != key_cache.dtype:
        raise ValueError("query must be [T, Hq, D] in the KV dtype")
    if tuple(out.shape) != (T, Hq, D) or out.dtype != key_cache.dtype:
        raise ValueError("out must be [T, Hq, D] in the KV dtype")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, MB]")
    S, MB = block_tables.shape
    if tuple(context_lens.shape) != (S,) or tuple(query_start.shape) != (S + 1,):
        raise ValueError("context_lens must be [S] and query_start [S+1]")
    rc = lib().pa_prefill_attention(
        _dev(out, "out"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), S, T, Hq, Hkv, D, bs, NB, MB,
        int(max_query_len), float(scale), dt, _stream(stream))
    _check(rc, "pa_prefill_attention")


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode
# ---------------------------------------------------------------------------
CASCADE_ITEM_INTS = 21
CASCADE_INFO_INTS = 6


class CascadePlan:
    """A plan from ``pa_cascade_plan``: ``plan`` (host int32: seq_start[S],
    slot_base[S], then n_items work items of 21 ints: table sequence, token
    start, token end, slot (-1 = direct output), member count, members) and
    its sizes."""

    def __init__(self, S: int, plan: np.ndarray, info: np.ndarray):
        self.S = S
        self.plan = plan
        self.n_items, self.slots_max, self.suffix_parts = (int(x) for x in info[:3])
        self.prefix_rows, self.saved_rows = int(info[4]), int(info[5])
        self._dev = None

    @property
    def seq_start(self) -> np.ndarray:
        return self.plan[:self.S]

    @property
    def slot_base(self) -> np.ndarray:
        return self.plan[self.S:2 * self.S]

    @property
    def items(self) -> np.ndarray:
        return self.plan[2 * self.S:].reshape(-1, CASCADE_ITEM_INTS)

    def device(self, device="cuda") -> torch.Tensor:
        """The plan as a device tensor, copied once (asynchronously on the
        current stream, through newly allocated pinned memory)."""
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if self._dev is None or self._dev.device != dev:
            src = self.plan if self.plan.size else np.zeros(1, dtype=np.int32)
            self._dev = torch.from_numpy(src).pin_memory().to(dev, non_blocking=True)
        return self._dev


def pa_cascade_plan(block_tables: np.ndarray, context_lens: np.ndarray, bs: int, Hq: int,
                    Hkv: int, partition_tokens: int = 0, prefix_tokens: int = 0) -> CascadePlan:
    """Plan the shared-prefix decode of a batch from its host block tables
    ([S, MB] int32) and context lengths ([S] int32)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or cl.shape != (bt.shape[0],):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    S, MB = bt.shape
    info = np.zeros(CASCADE_INFO_INTS, dtype=np.int32)
    pi32 = lambda a: a.ctypes.data_as(_p_i32)
    args = (pi32(bt), pi32(cl), S, MB, bs, Hq, Hkv, partition_tokens, prefix_tokens)
    rc = lib().pa_cascade_plan(*args, None, 0, pi32(info))
    if rc != PA_ERR_WORKSPACE:
        _check(rc, "pa_cascade_plan")
    plan = np.zeros(int(info[3]), dtype=np.int32)
    _check(lib().pa_cascade_plan(*args, pi32(plan), plan.size, pi32(info)), "pa_cascade_plan")
    return CascadePlan(S, plan, info)


def pa_cascade_workspace_bytes(S: int, Hq: int, D: int, slots_max: int) -> int:
    return int(lib().pa_cascade_workspace_bytes(S, Hq, D, slots_max))


def make_cascade_workspace(S: int, Hq: int, D: int, plan: CascadePlan,
                           device="cuda") -> Optional[torch.Tensor]:
    n = pa_cascade_workspace_bytes(S, Hq, D, plan.slots_max)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pa_decode_cascade(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, plan: CascadePlan, max_context_len: int,
                      scale: float, partition_tokens: int = 0,
                      workspace: Optional[torch.Tensor] = None,
                      key: Optional[torch.Tensor] = None, value: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Decode attention along a shared-prefix plan; with ``key``/``value``
    ([S, Hkv, D]) the new token is stored as in ``pa_decode_step``."""
    dt = _kv_dtype(key_cache)
    NB, Hkv, bs, D = key_cache.shape
    S, Hq, Dq = query.shape
    if Dq != D or query.dtype != key_cache.dtype:
        raise ValueError("query must be [S, Hq, D] in the KV dtype")
    if tuple(out.shape) != (S, Hq, D) or out.dtype != key_cache.dtype:
        raise ValueError("out must be [S, Hq, D] in the KV dtype")
    if (key is None) != (value is None):
        raise ValueError("give both key and value, or neither")
    kp = vp = None
    if key is not None:
        for name, t in (("key", key), ("value", value)):
            if tuple(t.shape) != (S, Hkv, D) or t.dtype != key_cache.dtype:
                raise ValueError(f"{name} must be [S, {Hkv}, {D}] {key_cache.dtype}")
        kp, vp = _dev(key, "key"), _dev(value, "value")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, MB]")
    if tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be [S]")
    if plan.S != S:
        raise ValueError("plan was built for another batch")
    MB = block_tables.shape[1]
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    pd = plan.device(query.device)
    rc = lib().pa_decode_cascade(
        _dev(out, "out"), _dev(query, "query"), kp, vp, _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), _dev(pd, "plan", torch.int32),
        plan.n_items, plan.slots_max, S, Hq, Hkv, D, bs, NB, MB,
        int(max_context_len), float(scale), int(partition_tokens), ws_ptr, ws_bytes, dt,
        _stream(stream))
    _check(rc, "pa_decode_cascade")


def pa_probe_read_bandwidth(src: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Diagnostic streaming read of all of ``src`` (device, any dtype, size a
    multiple of 16 bytes); ``out`` is a device int32 buffer of at least 256
    words that receives one folded word per thread."""
    nbytes = src.numel() * src.element_size()
    rc = lib().pa_probe_read_bandwidth(_dev(src, "src"), nbytes, _dev(out, "out", torch.int32),
                                       out.numel(), _stream(stream))
    _check(rc, "pa_probe_read_bandwidth")


def pa_copy_blocks(key_caches: Sequence[torch.Tensor], value_caches: Sequence[torch.Tensor],
                   block_mapping, stream=None) -> None:
    """Copy-on-write copies: for each (src, dst) in ``block_mapping`` (host
    int64 [n, 2]), block dst of every layer's K and V pool becomes a copy of
    block src."""
    L = len(key_caches)
    if len(value_caches) != L:
        raise ValueError("one value pool per key pool")
    pairs = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    n = pairs.shape[0]
    if L == 0 or n == 0:
        return
    ref = key_caches[0]
    NB = ref.shape[0]
    block_bytes = ref[0].numel() * ref.element_size()
    for t in list(key_caches) + list(value_caches):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("all pools must have one shape and dtype")
    kp = (_c_p * L)(*[_dev(t, "key_caches") for t in key_caches])
    vp = (_c_p * L)(*[_dev(t, "value_caches") for t in value_caches])
    rc = lib().pa_copy_blocks(kp, vp, L, pairs.ctypes.data_as(_p_i64), n, NB, block_bytes,
                              _stream(stream))
    _check(rc, "pa_copy_blocks")


# ---------------------------------------------------------------------------
# host allocator
# ---------------------------------------------------------------------------
class Allocator:
    """Host block allocator (C++): free list, refcounts, copy-on-write fork,
    prefix registry for sharing across requests."""

    def __init__(self, num_blocks: int, bs: int, init_order=None):
        L = lib()
        order = None
        if init_order is not None:
            self._order = np.ascontiguousarray(np.asarray(init_order, dtype=np.int32))
            if self._order.shape != (num_blocks,):
                raise ValueError("init_order must have num_blocks entries")
            order = self._order.ctypes.data_as(_p_i32)
        self._h = L.pa_alloc_create(num_blocks, bs, order)
        if not self._h:
            raise PaError(PA_ERR_INVALID, "pa_alloc_create")
        self.num_blocks = num_blocks
        self.bs = bs

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_alloc_destroy(h)
            self._h = None

    def num_free(self) -> int:
        return lib().pa_alloc_num_free(self._h)

    def refcount(self, block: int) -> int:
        return lib().pa_alloc_refcount(self._h, block)

    def create(self, seq_id: int) -> None:
        _check(lib().pa_seq_create(self._h, seq_id), "pa_seq_create")

    def append(self, seq_id: int):
        """(slot, cow_src, cow_dst) for the sequence's next token."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_seq_append(self._h, seq_id, ctypes.byref(slot), ctypes.byref(src),
                                   ctypes.byref(dst)), "pa_seq_append")
        return slot.value, src.value, dst.value

    def append_n(self, seq_id: int, n: int):
        """(slots[n] int64, cow_src, cow_dst)."""
        slots = np.empty(n, dtype=np.int64)
        src, dst = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_seq_append_n(self._h, seq_id, n, slots.ctypes.data_as(_p_i64),
                                     ctypes.byref(src), ctypes.byref(dst)), "pa_seq_append_n")
        return slots, src.value, dst.value

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pa_seq_fork(self._h, parent, child), "pa_seq_fork")

    def free(self, seq_id: int) -> None:
        _check(lib().pa_seq_free(self._h, seq_id), "pa_seq_free")

    def seq_len(self, seq_id: int) -> int:
        return lib().pa_seq_len(self._h, seq_id)

    def seq_blocks(self, seq_id: int) -> list:
        n = lib().pa_seq_num_blocks(self._h, seq_id)
        if n < 0:
            raise PaError(PA_ERR_INVALID, "pa_seq_num_blocks")
        buf = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().pa_seq_blocks(self._h, seq_id, buf.ctypes.data_as(_p_i32), n),
               "pa_seq_blocks")
        return buf[:n].tolist()

    def build_batch(self, seq_ids, MB: int):
        """(block_tables int32 [S, MB] padded with -1, context_lens int32 [S]), host."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        S = ids.shape[0]
        tables = np.empty((S, MB), dtype=np.int32)
        lens = np.empty(S, dtype=np.int32)
        _check(lib().pa_build_batch(self._h, ids.ctypes.data_as(_p_i64), S, MB,
                                    tables.ctypes.data_as(_p_i32), lens.ctypes.data_as(_p_i32)),
               "pa_build_batch")
        return tables, lens

    # -- prefix registry (sharing across requests) --------------------------
    @staticmethod
    def _keys(keys) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(keys, dtype=np.uint64).reshape(-1))

    def prefix_publish(self, seq_id: int, keys) -> int:
        """Register the sequence's first len(keys) full blocks; returns the
        number of new entries."""
        k = self._keys(keys)
        added = ctypes.c_int32()
        _check(lib().pa_prefix_publish(self._h, seq_id, k.ctypes.data_as(_p_u64), k.size,
                                       ctypes.byref(added)), "pa_prefix_publish")
        return added.value

    def create_prefixed(self, seq_id: int, keys) -> int:
        """New sequence starting with the registered blocks of the longest
        run of present keys; returns that run's length in blocks."""
        k = self._keys(keys)
        matched = ctypes.c_int32()
        _check(lib().pa_seq_create_prefixed(self._h, seq_id, k.ctypes.data_as(_p_u64), k.size,
                                            ctypes.byref(matched)), "pa_seq_create_prefixed")
        return matched.value

    def prefix_evict(self, keys) -> int:
        k = self._keys(keys)
        removed = ctypes.c_int32()
        _check(lib().pa_prefix_evict(self._h, k.ctypes.data_as(_p_u64), k.size,
                                     ctypes.byref(removed)), "pa_prefix_evict")
        return removed.value

    def prefix_size(self) -> int:
        return lib().pa_prefix_size(self._h)

    def export(self):
        """(refcounts [NB], free blocks in hand-out order)."""
        ref = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        free = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_alloc_export(self._h, ref.ctypes.data_as(_p_i32),
                                     free.ctypes.data_as(_p_i32), ctypes.byref(n)),
               "pa_alloc_export")
        return ref[:self.num_blocks].tolist(), free[:n.value].tolist()
