#!/usr/bin/env python3
"""Benchmark: one decode step of the paged KV path on one MI355X.

A step is the whole hot path over one batch: the cache write of each
sequence's new token and paged decode attention over its context.  It is
timed in both of the library's forms, as two calls (pa_reshape_and_cache,
then pa_decode_attention) and as the fused pa_decode_step (one launch),
alternating over three rounds of exactly K steps each; each form's median
is kept and the step is quoted on the faster (``step`` names it), the other
reported beside it.
Inputs are seeded synthetic data already resident in HBM; slots and block
tables come from the library's host allocator before the timed region.

Default run (no --workload): a launcher that makes no GPU call itself and
runs every measurement in a child process of its own, one after another:
  * the headline, the LLaMA-13B-shaped decode layer (128 sequences, 40 heads
    of 128, bfloat16 KV, block size 16, context lengths lognormal with median
    700, sigma 0.5, at most 2048), with the read-bandwidth probes and the CPU
    oracle baseline;
  * the block-size sweep of that batch (8, 32, 64, 128), one process each;
  * every other workload (tiny, LLaMA-7B-shaped, shared-prefix parallel
    sampling at 504- and 512-token prompts, long-context grouped-query), each
    with its own oracle baseline;
  * paged prefill of 16 LLaMA-13B-shaped prompts, with its oracle baseline.
One JSON line merges them: the headline's fields at the top level, the sweep
under ``sweep``, the others under ``configs``, the prefill under
``prefill``.  ``value`` is algorithmic KV
bytes (every attended token's K and V row once per head) per second of whole
step; ``roofline`` prices the attention launch alone (its average duration
from HIP events around it) against the 8 TB/s HBM peak;
``cpu_baseline`` times the float64 CPU oracle on the same workload.

    python bench.py [--steps K] [--warmup W] [--bs 16] [--no-sweep]
    python bench.py --workload NAME [...]   # one workload, in this process
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_llama13b_bs16.json")
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_198_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_device.h")]
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_llama13b.json")
PREFILL_SRCS = [os.path.join(ROOT, "paged_kv_cache_198_amd", "csrc", f)
                for f in ("pa_prefill.hip", "pa_mfma.h", "pa_device.h")]
WORKLOADS = ["llama13b", "llama7b", "long_gqa", "tiny", "shared_prefix", "system_prompt", "beam",
             "prefill"]


def source_sha(srcs) -> str:
    """Hash of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in srcs:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_source_sha() -> str:
    """Hash of the sources the VALU decode kernel is built from."""
    return source_sha(DECODE_SRCS)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=WORKLOADS,
                    help="time this workload in this process (default: run the headline, the "
                         "block-size sweep and the other workloads, each in a child process)")
    ap.add_argument("--bs", type=int, default=16)
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition tokens (0 = single pass, -1 = library default for the shape)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prompt-len", type=int, default=504,
                    help="shared_prefix: prompt tokens (504 leaves the last shared block "
                         "half full, so forks copy it; 512 fills it)")
    ap.add_argument("--prefix-tokens", type=int, default=0,
                    help="shared_prefix / system_prompt: tokens per shared-prefix work item "
                         "(0 = whole prefix)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="default run: skip the block-size sweep and the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work per workload for the CPU baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the plain HBM probe")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def default_partition(workload: str) -> int:
    """Partition size per workload: the long-context batch has only S*Hkv = 64
    (sequence, KV head) pairs, so it is split into 512-token partitions to
    fill the chip; the 7B batch's short lognormal contexts are split at 512
    tokens too, which evens out its workgroups; the others run in one pass."""
    from paged_kv_cache_198_amd import synth
    return synth.CONFIGS[workload]["partition_tokens"]


class Step:
    """Device state of one decode step, built once."""

    def __init__(self, pa, synth, torch, bs, seed, partition, workload="llama13b"):
        self.torch = torch
        self.pa = pa
        over = {"bs": bs} if workload == "llama13b" else {}
        w = synth.make_decode(workload, seed=seed, device="cuda", **over)
        self.w = w
        alloc = pa.Allocator(w.NB, w.bs, init_order=w.block_order)
        step = np.empty(w.S, dtype=np.int64)
        for s in range(w.S):
            alloc.create(s)
            slots, _, _ = alloc.append_n(s, int(w.context_lens[s]))
            step[s] = slots[-1]
        tables, lens = alloc.build_batch(list(range(w.S)), w.MB)
        self.slots = torch.from_numpy(step).cuda()
        self.tables = torch.from_numpy(tables).cuda()
        self.lens = torch.from_numpy(lens).cuda()
        self.max_ctx = int(lens.max())
        self.part = default_partition(workload) if partition < 0 else partition
        self.out = torch.empty(w.S, w.Hq, w.D, dtype=w.q.dtype, device="cuda")
        self.ws = pa.make_workspace(w.S, w.Hq, w.D, self.max_ctx, self.part)
        self.kv_bytes = int(np.sum(lens.astype(np.int64))) * 2 * w.Hkv * w.D * w.elem_bytes

    def write(self):
        w = self.w
        self.pa.pa_reshape_and_cache(w.new_key, w.new_value, w.key_cache, w.value_cache,
                                     self.slots)

    def attend(self):
        w = self.w
        self.pa.pa_decode_attention(self.out, w.q, w.key_cache, w.value_cache, self.tables,
                                    self.lens, self.max_ctx, w.scale, self.part, self.ws)

    def fused(self):
        w = self.w
        self.pa.pa_decode_step(self.out, w.q, w.new_key, w.new_value, w.key_cache,
                               w.value_cache, self.tables, self.lens, self.max_ctx, w.scale,
                               self.part, self.ws)

    def kernel_time(self, reps, warmup):
        """Average duration of the attention launch (pa_decode_attention;
        with partitions, its main pass and the reduce): ``reps`` launches back
        to back on the launch stream between two events, so the figure is
        the launch's own duration plus the gap to the next.  The pools are
        not written in between; the launch reads the same bytes either way.
        Returns milliseconds."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.attend()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            self.attend()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def run(self, steps, warmup, fused=True):
        """Time ``steps`` decode steps between two events on the launch stream
        (no events inside the region, so nothing sits between launches).
        Returns (ms per step, wall seconds)."""
        torch = self.torch
        step = self.fused if fused else (lambda: (self.write(), self.attend()))
        for _ in range(warmup):
            step()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for _ in range(steps):
            step()
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(stop) / steps, wall


def kernel_name(st) -> str:
    """The attention launch of pa_decode_attention for this workload."""
    w = st.w
    mfma = w.dtype in ("bf16", "f16") and w.D == 128 and w.Hq // w.Hkv == 8
    k = "pa::decode_gqa_mfma_kernel" if mfma else "pa::decode_kernel"
    parts = -(-st.max_ctx // st.part) if st.part else 1
    red = "" if parts < 2 else (" + reduce_wide_kernel" if parts >= 16 else " + reduce_kernel")
    return k + red + " (pa_decode_attention)"


def describe(name, w) -> str:
    from paged_kv_cache_198_amd import synth
    law = synth.CONFIGS[name]["lengths"]
    lens = (f"lognormal(median {law[1]}, sigma {law[2]}) in [{law[3]}, {law[4]}]"
            if law[0] == "lognormal" else f"uniform in [{law[1]}, {law[2]}]")
    title = {"llama13b": "LLaMA-13B-shaped decode layer", "llama7b": "LLaMA-7B-shaped decode layer",
             "long_gqa": "long-context GQA decode (one GPU's share of a 70B-shaped layer)",
             "tiny": "tiny paged decode"}[name]
    return (f"{title}: S={w.S}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, {w.dtype} KV, block_size {w.bs}, "
            f"ctx {lens}, {w.NB}-block pool shuffled, 1 new token per sequence")


def traffic_bytes(path=TRAFFIC_FILE, srcs=DECODE_SRCS):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_sha(srcs):
        return None
    return float(t["bytes_per_launch"])


def host_threads():
    """(host cores this process may run on, BLAS threads numpy uses)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = 1
    return cores, int(blas)


def timed_reps(fn, budget_s, max_reps=5):
    """Run ``fn`` (returns its own seconds) at least once and until about
    ``budget_s`` seconds are spent; the median and the count."""
    times = [fn()]
    while sum(times) < budget_s and len(times) < max_reps:
        times.append(fn())
    return float(np.median(times)), len(times)


def baseline_record(kv_bytes, secs, reps, what):
    cores, blas = host_threads()
    return {"value": kv_bytes / secs / 1e9, "unit": "GB/s", "cores": blas, "kind": "oracle",
            "s_per_step": secs, "reps": reps, "host_cores": cores, "blas_threads": blas,
            "sample": what + "; float64 numpy (gathers single-threaded, matrix-vector "
                             f"products through BLAS with up to {blas} threads)"}


class OracleStep:
    """The float64 oracle on the host over the same decode step: the cache
    write of every sequence's new token (slots from the oracle's own walk of
    the block tables) and the attention of every sequence, on host copies of
    the blocks the batch references.

    The host inputs are copied when this object is built, before any GPU
    step touches the pools.  ``time`` repeats one whole step for about
    ``budget_s`` seconds (the first sequences only when a whole step would
    take far longer; the record says how many) and compares the oracle's
    output with the GPU's on the same sequences."""

    def __init__(self, step, budget_s=8.0):
        import oracle.decode as od
        self.od = od
        self.step = step
        self.budget_s = budget_s
        w = step.w
        few = list(range(min(8, w.S)))
        hf = self._host_inputs(few)
        per_tok = min(self._run(hf)[0], self._run(self._host_inputs(few))[0]) / max(
            int(np.sum(w.context_lens[few])), 1)
        est = per_tok * float(np.sum(w.context_lens))
        if est <= 4 * budget_s:
            self.seqs = list(range(w.S))
            self.what = f"one whole decode step ({w.S} sequences)"
        else:
            csum = np.cumsum(w.context_lens.astype(np.int64))
            n = int(max(1, np.searchsorted(csum, budget_s / per_tok)))
            self.seqs = list(range(min(n, w.S)))
            self.what = (f"the first {len(self.seqs)} of {w.S} sequences of one decode step (a "
                         f"whole step would take about {est:.0f} s); value scaled by their KV bytes")
        self.h = self._host_inputs(self.seqs)

    def _host_inputs(self, seqs):
        from paged_kv_cache_198_amd import synth
        w = self.step.w
        torch = self.step.torch
        need = [-(-int(w.context_lens[s]) // w.bs) for s in seqs]
        blocks = np.unique(np.concatenate([w.block_tables[s, :n] for s, n in zip(seqs, need)]))
        remap = np.full(w.NB, -1, dtype=np.int64)
        remap[blocks] = np.arange(len(blocks))
        idx = torch.from_numpy(blocks.astype(np.int64)).to(w.q.device)
        sel = torch.tensor(seqs, device=w.q.device)
        return dict(
            kc=synth.to_numpy_storage(w.key_cache.index_select(0, idx)),
            vc=synth.to_numpy_storage(w.value_cache.index_select(0, idx)),
            tab=np.where(w.block_tables[seqs] >= 0,
                         remap[np.maximum(w.block_tables[seqs], 0)], -1),
            lens=w.context_lens[seqs], q=synth.to_numpy_storage(w.q.index_select(0, sel)),
            nk=synth.to_numpy_storage(w.new_key.index_select(0, sel)),
            nv=synth.to_numpy_storage(w.new_value.index_select(0, sel)))

    def _run(self, h):
        od, w = self.od, self.step.w
        t0 = time.perf_counter()
        slots = [od.slot_of(h["tab"][i], int(h["lens"][i]) - 1, w.bs) for i in range(len(h["lens"]))]
        od.reshape_and_cache(h["nk"], h["nv"], h["kc"], h["vc"], slots, inplace=True)
        out = od.paged_decode(h["q"], h["kc"], h["vc"], h["tab"], h["lens"], w.scale, w.dtype)
        return time.perf_counter() - t0, out

    def time(self, gpu_out=None):
        """The baseline record; ``gpu_out`` is the GPU's output of the same
        step ([S, Hq, D], any device), compared on the sampled sequences."""
        from paged_kv_cache_198_amd import synth
        w = self.step.w
        kv = int(np.sum(w.context_lens[self.seqs].astype(np.int64))) * 2 * w.Hkv * w.D * w.elem_bytes
        outs = []

        def once():
            t, o = self._run(self.h)
            outs.append(o)
            return t

        secs, reps = timed_reps(once, self.budget_s)
        rec = baseline_record(kv, secs, reps, f"{self.what}, median of {reps}")
        if gpu_out is not None:
            got = self.od.widen(synth.to_numpy_storage(gpu_out.index_select(
                0, self.step.torch.tensor(self.seqs, device=gpu_out.device))), w.dtype)
            rec["max_abs_err_vs_gpu"] = float(np.max(np.abs(got - outs[-1])))
        return rec


def max_err_vs_gpu(ref, gpu_out, dtype):
    """Largest difference between an oracle output and the GPU's."""
    import oracle.decode as od
    from paged_kv_cache_198_amd import synth
    got = od.widen(synth.to_numpy_storage(gpu_out), dtype)
    return float(np.max(np.abs(got - ref)))


def cpu_baseline_shared_prefix(sc, budget_s=8.0, gpu_out=None):
    """The oracle's own drive of the parallel-sampling script (its
    allocator, copy-on-write copies and cache writes, untimed) up to the
    decode step, then that step timed once: every sample's next slot and
    copy-on-write copies, the cache write of the new tokens and the attention
    of all samples."""
    import oracle.alloc as oa
    import oracle.decode as od
    from paged_kv_cache_198_amd import synth
    kc = synth.to_numpy_storage(sc.key_cache).copy()
    vc = synth.to_numpy_storage(sc.value_cache).copy()
    pk, pv = synth.to_numpy_storage(sc.prompt_k), synth.to_numpy_storage(sc.prompt_v)
    tk, tv = synth.to_numpy_storage(sc.tail_k), synth.to_numpy_storage(sc.tail_v)
    sk, sv = synth.to_numpy_storage(sc.step_k), synth.to_numpy_storage(sc.step_v)
    q = synth.to_numpy_storage(sc.q)
    alloc = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    for i in range(sc.prompts):
        sid = sc.seq_id(i, 0)
        alloc.create(sid)
        slots = [alloc.append(sid)[0] for _ in range(sc.prompt_len)]
        od.reshape_and_cache(pk[i], pv[i], kc, vc, slots, inplace=True)
        for j in range(1, sc.samples):
            alloc.fork(sid, sc.seq_id(i, j))

    def advance(who, k, v):
        pairs, slots = [], []
        for s in who:
            slot, src, dst = alloc.append(s)
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        od.copy_blocks([kc], [vc], pairs, inplace=True)
        od.reshape_and_cache(k, v, kc, vc, slots, inplace=True)

    for t in range(int(sc.tails.max()) if sc.S else 0):
        who = [s for s in range(sc.S) if t < sc.tails[s]]
        advance(who, tk[who, t], tv[who, t])
    seqs = list(range(sc.S))
    t0 = time.perf_counter()
    advance(seqs, sk, sv)
    MB = max(-(-alloc.seq_len(s) // sc.bs) for s in seqs)
    tables, lens = alloc.build_batch(seqs, MB)
    ref = od.paged_decode(q, kc, vc, np.array(tables), np.array(lens), sc.scale, sc.dtype)
    secs = time.perf_counter() - t0
    kv = int(np.sum(np.asarray(lens, dtype=np.int64))) * 2 * sc.Hkv * sc.D * synth.ELEM_BYTES[sc.dtype]
    rec = baseline_record(kv, secs, 1, f"one whole decode step ({sc.S} samples, logical bytes: "
                                       "each sample's whole context), the state built by the "
                                       "oracle's own allocator and cache writes beforehand")
    if gpu_out is not None:
        rec["max_abs_err_vs_gpu"] = max_err_vs_gpu(ref, gpu_out, sc.dtype)
    return rec


def cpu_baseline_system_prompt(sc, gpu_out=None):
    """The oracle's own drive of the system-prompt script (request 0 stores
    its prompt and publishes the system prompt's full blocks; every later
    request takes them from the oracle's registry and stores only its own
    tokens; untimed), then the decode step timed once: every request's next
    slot, the cache write of the new tokens and the attention of all
    requests.  The inputs are the script's own tensors, which no kernel of
    the library writes."""
    import oracle.alloc as oa
    import oracle.decode as od
    from paged_kv_cache_198_amd import synth
    kc = synth.to_numpy_storage(sc.key_cache).copy()
    vc = synth.to_numpy_storage(sc.value_cache).copy()
    alloc = oa.Allocator(sc.NB, sc.bs, init_order=sc.init_order)
    keys = sc.system_keys()
    for r in range(sc.requests):
        k, v = sc.prompt(r)
        k, v = synth.to_numpy_storage(k), synth.to_numpy_storage(v)
        m = 0
        if r == 0:
            alloc.create(0)
        else:
            m = alloc.create_prefixed(r, keys) * sc.bs
        slots = [alloc.append(r)[0] for _ in range(k.shape[0] - m)]
        od.reshape_and_cache(k[m:], v[m:], kc, vc, slots, inplace=True)
        if r == 0:
            alloc.publish(0, keys)
    seqs = list(range(sc.requests))
    sk, sv = synth.to_numpy_storage(sc.step_k), synth.to_numpy_storage(sc.step_v)
    q = synth.to_numpy_storage(sc.q)
    t0 = time.perf_counter()
    res = [alloc.append(r) for r in seqs]
    od.copy_blocks([kc], [vc], [(x[1], x[2]) for x in res if x[1] >= 0], inplace=True)
    od.reshape_and_cache(sk, sv, kc, vc, [x[0] for x in res], inplace=True)
    MB = max(-(-alloc.seq_len(r) // sc.bs) for r in seqs)
    tables, lens = alloc.build_batch(seqs, MB)
    ref = od.paged_decode(q, kc, vc, np.array(tables), np.array(lens), sc.scale, sc.dtype)
    secs = time.perf_counter() - t0
    kv = int(np.sum(np.asarray(lens, dtype=np.int64))) * 2 * sc.Hkv * sc.D * synth.ELEM_BYTES[sc.dtype]
    rec = baseline_record(kv, secs, 1, f"one whole decode step ({sc.requests} requests, logical "
                                       "bytes: each request's whole context), the state built "
                                       "by the oracle's own allocator, registry and cache writes")
    if gpu_out is not None:
        rec["max_abs_err_vs_gpu"] = max_err_vs_gpu(ref, gpu_out, sc.dtype)
    return rec


def read_probe(pa, torch, nbytes, grids, reps=10):
    """The library's plain streaming-read kernel over ``nbytes``, at each
    workgroup count in ``grids``: the read rate this machine reaches with the
    decode kernels' loads and no math.  Returns {grid: GB/s}."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    rates = {}
    for grid in grids:
        out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        pa.pa_probe_read_bandwidth(src, out)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            pa.pa_probe_read_bandwidth(src, out)
        e.record()
        torch.cuda.synchronize()
        rates[grid] = (nbytes // 2) * 2 * reps / (s.elapsed_time(e) * 1e-3) / 1e9
        del out
    del src
    torch.cuda.empty_cache()
    return rates


def hbm_probe(torch, gib=4, reps=10):
    """Plain device-memory rates on this machine from torch's own kernels: a copy
    (read + write) and a sum (read only) over ``gib`` GiB; context for the
    fraction of the 8 TB/s peak the decode kernel reaches."""
    n = gib << 30
    a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * n), ("sum", lambda: a.sum(), n)):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        out[f"torch_{name}_GBs"] = moved * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return out


def calibrate_copy(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def run_shared_prefix(args, pa, synth, torch):
    """Blocks shared between sequences, two workloads:
      shared_prefix  parallel sampling: 16 prompts x 4 samples forked from
                     each prompt (copy-on-write on divergence);
      system_prompt  64 requests whose prompts start with one 1024-token
                     system prompt, registered once and reused through the
                     prefix registry.
    Setup runs through the library's allocator and kernels; then every
    sequence reserves its next slot and K decode steps are timed twice on the
    same state: the plain fused step (every sequence reads its whole context)
    and the shared-prefix step (pa_cascade_plan + pa_decode_cascade: shared
    blocks read once per group).  Logical bytes count each sequence's whole
    context."""
    import time
    from paged_kv_cache_198_amd import engine
    if args.workload == "system_prompt":
        sc = synth.make_system_prompt(seed=args.seed, device="cuda")
        kv = engine.build_system_prompt(sc)
        desc = (f"system prompt shared across requests: {sc.requests} requests, "
                f"{sc.system_len}-token system prompt registered once, own prompt uniform "
                f"[{synth.SYSTEM_PROMPT['own'][0]}, {synth.SYSTEM_PROMPT['own'][1]}] tokens, "
                f"Hq={sc.Hq}, Hkv={sc.Hkv}, D={sc.D}, {sc.dtype}, block_size {sc.bs}, "
                f"{sc.NB}-block pool")
        extra = {"system_len": sc.system_len}
    else:
        sc = synth.make_shared_prefix(seed=args.seed, device="cuda", prompt_len=args.prompt_len)
        kv = engine.build_shared_prefix(sc)
        desc = (f"shared-prefix parallel sampling: {sc.prompts} prompts x {sc.samples} samples, "
                f"Hq=Hkv={sc.Hkv}, D={sc.D}, {sc.dtype}, block_size {sc.bs}, prompt "
                f"{sc.prompt_len} tokens in shared blocks, tails uniform in [0, 256], "
                f"{sc.NB}-block pool")
        extra = {"prompt_len": sc.prompt_len}
    S = sc.q.shape[0]
    fork_copies = kv.copies
    seqs = list(range(S))
    _, pairs = kv.reserve(seqs)
    MB = max(-(-kv.alloc.seq_len(s) // sc.bs) for s in seqs)
    tables_h, lens_h32 = kv.alloc.build_batch(seqs, MB)
    tables = torch.from_numpy(tables_h).to("cuda")
    lens = torch.from_numpy(lens_h32).to("cuda")
    mx = int(lens_h32.max())
    out = torch.empty(S, sc.Hq, sc.D, dtype=sc.q.dtype, device="cuda")
    t0 = time.perf_counter()
    plan = pa.pa_cascade_plan(tables_h, lens_h32, sc.bs, sc.Hq, sc.Hkv, 0, args.prefix_tokens)
    plan_us = (time.perf_counter() - t0) * 1e6
    ws = pa.make_cascade_workspace(S, sc.Hq, sc.D, plan)

    def plain():
        pa.pa_decode_step(out, sc.q, sc.step_k, sc.step_v, kv.key_cache, kv.value_cache,
                          tables, lens, mx, sc.scale, 0, None)

    def cascade():
        pa.pa_decode_cascade(out, sc.q, kv.key_cache, kv.value_cache, tables, lens, plan, mx,
                             sc.scale, 0, ws, key=sc.step_k, value=sc.step_v)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    plain_ms = timed(plain)
    step_ms = timed(cascade)
    eb = synth.ELEM_BYTES[sc.dtype]
    row = 2 * sc.Hkv * sc.D * eb                           # K and V bytes of one token
    lens_h = lens_h32.astype(np.int64)
    logical = int(lens_h.sum()) * row
    items = plan.items
    cascade_rows = int((items[:, 2] - items[:, 1]).sum())   # prefix pieces once, every suffix
    cascade_bytes = cascade_rows * row
    unique_blocks = kv.used_blocks()
    block_bytes = sc.bs * sc.Hkv * sc.D * eb
    unique = unique_blocks * 2 * block_bytes
    private_blocks = kv.logical_blocks(seqs)
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    res = {
        "metric": "decode-attention KV GB/s (logical: each sequence's whole context) + us/step, "
                  f"{args.workload.replace('_', '-')} batch",
        "value": gbs(logical, step_ms), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "us_per_step": step_ms * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sc.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, uniform lengths)",
        "config": {"workload": desc, "S": S, "seed": args.seed,
                   "prefix_tokens": args.prefix_tokens, **extra,
                   "logical_kv_bytes": logical, "cascade_kv_bytes": cascade_bytes,
                   "unique_kv_bytes": unique},
        "roofline": {"bound": "hbm", "achieved": gbs(cascade_bytes, step_ms),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs(cascade_bytes, step_ms) / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "whole cascade step (work-item kernel + partition reduce)",
                     "note": "achieved counts the bytes the cascade must read: each shared "
                             "prefix once per group, every suffix once"},
        "plain_fused_step": {"us": plain_ms * 1e3, "logical_GBs": gbs(logical, plain_ms),
                             "speedup_of_cascade": plain_ms / step_ms,
                             "kernel": "pa::decode_kernel (pa_decode_step, fused cache write)"},
        "plan": {"items": plan.n_items, "slots_max": plan.slots_max,
                 "prefix_rows": plan.prefix_rows, "saved_rows": plan.saved_rows,
                 "host_plan_us": plan_us},
        "sharing": {"blocks_used": unique_blocks, "blocks_if_private": private_blocks,
                    "memory_saving": 1.0 - unique_blocks / private_blocks,
                    "cow_copies_at_fork": fork_copies, "cow_pairs_this_step": len(pairs)},
        "cpu_baseline": None,
    }
    if args.workload == "system_prompt":
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline_system_prompt(sc, out)
        return res
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_shared_prefix(sc, args.cpu_budget, out)

    # copy-on-write block copies across the layers of a 40-layer model: the
    # fork-time divergence of this batch (one pair per sample that writes
    # into its prompt's half-filled last block) copied in every layer
    L, nb_l = 40, 512
    pools_k = [torch.empty(nb_l, sc.Hkv, sc.bs, sc.D, dtype=sc.q.dtype, device="cuda")
               for _ in range(L)]
    pools_v = [torch.empty_like(pools_k[0]) for _ in range(L)]
    n_pairs = max(fork_copies, 1)
    perm = np.random.default_rng(args.seed).permutation(nb_l)
    cow = np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], axis=1)
    for _ in range(3):
        pa.pa_copy_blocks(pools_k, pools_v, cow)
    torch.cuda.synchronize()
    start.record()
    for _ in range(20):
        pa.pa_copy_blocks(pools_k, pools_v, cow)
    stop.record()
    torch.cuda.synchronize()
    cow_ms = start.elapsed_time(stop) / 20
    cow_bytes = 2 * n_pairs * L * 2 * block_bytes          # read + write, K and V
    res["cow_copy"] = {"pairs": n_pairs, "layers": L, "us": cow_ms * 1e3,
                       "GBs": cow_bytes / (cow_ms * 1e-3) / 1e9}
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / f16 matrix-core peak


def run_prefill(args, pa, synth, torch):
    """Prefill of a LLaMA-13B-shaped attention layer: 16 prompts with
    lognormal lengths (median 700, in [16, 2048]), bf16, bs 16.  One step =
    the cache write of every prompt token (pa_reshape_and_cache) + causal
    paged attention over the prompts (pa_prefill_attention).  Algorithmic
    flops per step = sum over prompt rows and query heads of 4 D (p + 1)
    (two products over the p + 1 attended keys)."""
    w = synth.make_prefill(seed=args.seed, device="cuda", bs=args.bs)
    # slots and tables from the library's allocator: each prompt grows to its
    # length in a pool handing out blocks in the workload's order
    alloc = pa.Allocator(w.NB, w.bs, init_order=w.block_order)
    rows = []
    for s in range(w.S):
        alloc.create(s)
        sl, _, _ = alloc.append_n(s, int(w.context_lens[s]))
        rows.append(sl[len(sl) - int(w.chunk_lens[s]):])
    tables_h, _ = alloc.build_batch(list(range(w.S)), w.MB)
    slots = torch.from_numpy(np.concatenate(rows)).to("cuda")
    tables = torch.from_numpy(tables_h).to("cuda")
    lens = torch.from_numpy(w.context_lens).to("cuda")
    qs = torch.from_numpy(w.query_start).to("cuda")
    kc, vc = w.key_cache, w.value_cache
    out = torch.empty_like(w.q)
    mq = int(w.chunk_lens.max())
    stream = torch.cuda.current_stream()
    # the oracle's host inputs, copied before any GPU step writes the pools
    oracle_in = None if args.no_cpu_baseline else {
        "q": synth.to_numpy_storage(w.q), "nk": synth.to_numpy_storage(w.new_key),
        "nv": synth.to_numpy_storage(w.new_value), "kc": synth.to_numpy_storage(kc).copy(),
        "vc": synth.to_numpy_storage(vc).copy()}

    def step():
        pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc, slots)
        pa.pa_prefill_attention(out, w.q, kc, vc, tables, lens, qs, mq, w.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # The attention kernel inside the step: events around it, after each
    # step's cache write (which streams the prompts' K/V through the caches
    # first, as a real prefill does).
    reps = max(20, args.steps // 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        pa.pa_reshape_and_cache(w.new_key, w.new_value, kc, vc, slots)
        e0.record(stream)
        pa.pa_prefill_attention(out, w.q, kc, vc, tables, lens, qs, mq, w.scale)
        e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / reps
    # and back to back, with the K/V left in the caches by the previous launch
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(reps):
        pa.pa_prefill_attention(out, w.q, kc, vc, tables, lens, qs, mq, w.scale)
    k1.record(stream)
    torch.cuda.synchronize()
    warm_ms = k0.elapsed_time(k1) / reps
    flops = 0
    for s in range(w.S):
        n, c = int(w.chunk_lens[s]), int(w.context_lens[s])
        keys = (c - n + 1 + c) * n // 2            # sum of (p + 1) over the chunk's rows
        flops += 4 * w.D * w.Hq * keys
    if args.calibrate_copy:
        calibrate_copy(torch)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    return {
        "metric": "prefill attention TFLOP/s (causal, algorithmic) + prompt tokens/s, "
                  "13B-shaped layer",
        "value": w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "us_per_step": ms * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, lognormal prompt lengths)",
        "config": {"workload": f"prefill: {w.S} prompts, lengths lognormal(median 700, sigma "
                               f"0.5) in [16, 2048] ({w.T} tokens), Hq=Hkv={w.Hkv}, D={w.D}, "
                               f"{w.dtype}, block_size {w.bs}, {w.NB}-block pool",
                   "tokens": w.T, "seed": args.seed, "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_bytes(PREFILL_TRAFFIC_FILE, PREFILL_SRCS)
                                if args.bs == 16 else None,
                     "kernel": "pa::prefill_kernel (pa_prefill_attention)",
                     "kernel_us": attn_ms * 1e3,
                     "note": "kernel_us: the attention launch inside the step, after the "
                             "cache write; back_to_back_us: repeated launches with K/V "
                             "still cached"},
        "back_to_back_us": warm_ms * 1e3,
        "cpu_baseline": None if oracle_in is None else cpu_baseline_prefill(
            w, oracle_in, out, args.cpu_budget),
    }


def cpu_baseline_prefill(w, h, gpu_out, budget_s=8.0):
    """The float64 oracle on the host over the same prefill step: the cache
    write of every prompt token (slots from the oracle's own walk of the
    block tables) and causal attention, on the inputs copied before the
    first GPU step.  All prompts when a step fits about ``budget_s``
    seconds, else the first ones (value scaled by their tokens).  Also the
    largest difference from the GPU's output on those prompts."""
    import oracle.decode as od
    from paged_kv_cache_198_amd import synth
    S = w.S
    n = w.chunk_lens.astype(np.int64)
    ctx = w.context_lens.astype(np.int64)
    slots = [od.slot_of(w.block_tables[s], int(p), w.bs)
             for s in range(S) for p in range(int(ctx[s] - n[s]), int(ctx[s]))]
    od.reshape_and_cache(h["nk"], h["nv"], h["kc"], h["vc"], slots, inplace=True)

    def run(seqs):
        t0 = time.perf_counter()
        o = od.paged_prefill(h["q"], h["kc"], h["vc"], w.block_tables, w.context_lens,
                             w.query_start, w.scale, w.dtype, seqs=seqs)
        return time.perf_counter() - t0, o

    # the cost of the first prompt sets the sample
    t_first, _ = run([0])
    per_tok = t_first / max(int(n[0]) ** 2, 1)           # causal work grows as n^2
    seqs, total = [], 0.0
    for s in range(S):
        est = per_tok * float(n[s]) ** 2
        if seqs and total + est > budget_s:
            break
        seqs.append(s)
        total += est
    secs, ref = run(seqs)
    toks = int(n[seqs].sum())
    rows = np.concatenate([np.arange(w.query_start[s], w.query_start[s + 1]) for s in seqs])
    got = od.widen(synth.to_numpy_storage(gpu_out)[rows], w.dtype)
    cores, blas = host_threads()
    sf = sum(4 * w.D * w.Hq * int((ctx[s] - n[s] + 1 + ctx[s]) * n[s] // 2) for s in seqs)
    what = (f"the whole prefill step ({S} prompts)" if len(seqs) == S else
            f"the first {len(seqs)} of {S} prompts ({toks} of {w.T} tokens); value scaled by "
            "their tokens")
    return {"value": toks / secs, "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "s_for_sample": secs, "tflops": sf / secs / 1e12, "host_cores": cores,
            "blas_threads": blas,
            "sample": what + "; float64 numpy, cache write untimed (done once before)",
            "max_abs_err_vs_gpu": float(np.max(np.abs(got - ref[rows])))}


BEAM_BENCH = dict(requests=16, width=4, layers=40, Hq=40, Hkv=40, D=128, dtype="bf16", bs=16,
                  NB=4096, prompt=(384, 640))


class _HostBeams:
    """The allocator side of a beam run without pools: the same creates,
    forks, frees and appends (engine.beam_reselect only forks and frees)."""

    def __init__(self, pa, num_blocks, bs):
        self.alloc = pa.Allocator(num_blocks, bs)

    def fork(self, parent, child):
        self.alloc.fork(parent, child)

    def free(self, seq_id):
        self.alloc.free(seq_id)


def run_beam(args, pa, synth, torch):
    """Beam search on a 40-layer, LLaMA-13B-shaped attention stack: 16
    requests x 4 beams whose prompts are shared by their beams.  One step =
    the beam selection (random parents: forks and frees in the allocator),
    every beam's next slot (copy-on-write copies batched over all 40 layers
    in one pa_copy_blocks call), then for each layer the new token's store
    and attention.  Timed from the same starting state twice: plain fused
    steps, and the shared-prefix path (one plan per step for all layers)."""
    import time
    from paged_kv_cache_198_amd import engine
    c = dict(BEAM_BENCH)
    # --bs picks the block size; the pool keeps the same token capacity
    c["NB"] = c["NB"] * c["bs"] // args.bs
    c["bs"] = args.bs
    R, W, L, bs = c["requests"], c["width"], c["layers"], c["bs"]
    dt = synth.KV_DTYPES[c["dtype"]]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed)
    rng = np.random.default_rng(args.seed)
    plens = rng.integers(c["prompt"][0], c["prompt"][1] + 1, size=R)
    total = args.warmup + args.steps
    choices = rng.integers(0, W, size=(total, R, W)).tolist()
    S = R * W
    # values do not change the work: one random prompt, token and query set
    pk = torch.randn(L, int(plens.max()), c["Hkv"], c["D"], generator=gen, device="cuda").to(dt)
    nk = torch.randn(L, S, c["Hkv"], c["D"], generator=gen, device="cuda").to(dt)
    q = torch.randn(L, S, c["Hq"], c["D"], generator=gen, device="cuda").to(dt)
    scale = float(np.float32(1.0 / np.sqrt(c["D"])))
    eb = synth.ELEM_BYTES[c["dtype"]]
    row = 2 * c["Hkv"] * c["D"] * eb

    def build():
        kv = engine.PagedKV(c["NB"], bs, c["Hkv"], c["D"], c["dtype"], device="cuda", layers=L,
                            init_order=np.random.default_rng(args.seed).permutation(c["NB"]))
        beams, nxt = [], R
        for r in range(R):
            n = int(plens[r])
            kv.prefill(r, pk[:, :n], pk[:, :n])
            group = [r]
            for _ in range(W - 1):
                kv.fork(r, nxt)
                group.append(nxt)
                nxt += 1
            beams.append(group)
        return kv, beams, nxt

    def run(cascade):
        kv, beams, nxt = build()
        torch.cuda.synchronize()
        stats = {"copies": 0, "logical": 0, "read": 0, "host_s": 0.0}
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        for t in range(total):
            if t == args.warmup:
                torch.cuda.synchronize()
                start.record()
            h0 = time.perf_counter()
            before = kv.copies
            beams, nxt = engine.beam_reselect(kv, beams, choices[t], nxt)
            flat = [b for g in beams for b in g]
            if cascade:
                _, plan = kv.step_cascade(q, flat, nk, nk, scale)
                read = int((plan.items[:, 2] - plan.items[:, 1]).sum())
            else:
                kv.step(q, flat, nk, nk, scale)
                read = None
            if t >= args.warmup:
                ctx = sum(kv.alloc.seq_len(b) for b in flat)
                stats["copies"] += kv.copies - before
                stats["logical"] += L * ctx * row
                stats["read"] += L * (ctx if read is None else read) * row
                stats["host_s"] += time.perf_counter() - h0
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        return ms, {k: v / args.steps for k, v in stats.items()}, kv, beams

    # the oracle's host inputs (layer 0), copied before any GPU step
    oracle_in = None if args.no_cpu_baseline else {
        "pk": synth.to_numpy_storage(pk[0]), "nk": synth.to_numpy_storage(nk[0]),
        "q": synth.to_numpy_storage(q[0])}
    plain_ms, plain_st, kv, _ = run(False)
    used_plain = kv.used_blocks()
    del kv
    torch.cuda.empty_cache()
    ms, st, kv, end_beams = run(True)
    held = kv.used_blocks() * bs
    host = _HostBeams(pa, c["NB"] * bs, 1)
    hbeams, hnext = [], R
    for r in range(R):
        host.alloc.create(r)
        host.alloc.append_n(r, int(plens[r]))
        group = [r]
        for _ in range(W - 1):
            host.fork(r, hnext)
            group.append(hnext)
            hnext += 1
        hbeams.append(group)
    for t in range(total):
        hbeams, hnext = engine.beam_reselect(host, hbeams, choices[t], hnext)
        for b in (b for g in hbeams for b in g):
            host.alloc.append(b)
    tree = c["NB"] * bs - host.alloc.num_free()
    gbs = lambda b, m: b / (m * 1e-3) / 1e9
    return {
        "metric": "beam-search decode step over 40 layers: KV GB/s (logical) + us/step",
        "value": gbs(st["logical"], ms), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "us_per_step": ms * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c["dtype"],
        "data": "synthetic (random K/V/q, random beam parents)",
        "config": {"workload": f"beam search: {R} requests x {W} beams, {L} layers, "
                               f"Hq=Hkv={c['Hkv']}, D={c['D']}, {c['dtype']}, block_size {bs}, "
                               f"prompts uniform [{c['prompt'][0]}, {c['prompt'][1]}], "
                               f"{c['NB']}-block pool per layer",
                   "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": gbs(st["read"], ms), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs(st["read"], ms) / HBM_PEAK_GBS,
                     "traffic": None,
                     "kernel": "whole beam step (copies + 40 x (item kernel + reduce))",
                     "note": "achieved counts the K/V bytes the cascade must read per step"},
        "per_step": {"cow_copies": st["copies"], "logical_kv_bytes": st["logical"],
                     "read_kv_bytes": st["read"], "host_us": st["host_s"] * 1e6,
                     # each copy moves a whole block of K and V in every layer
                     "cow_bytes_moved": st["copies"] * 2 * L * bs * c["Hkv"] * c["D"] * eb * 2},
        "plain_fused_step": {"us": plain_ms * 1e3, "logical_GBs": gbs(plain_st["logical"], plain_ms),
                             "host_us": plain_st["host_s"] * 1e6,
                             "speedup_of_cascade": plain_ms / ms},
        "blocks_used_per_layer": {"plain_run_end": used_plain, "cascade_run_end": kv.used_blocks()},
        "slots_per_layer_at_end": {
            "held": held, "beam_tree_tokens": tree,
            "waste": 1 - tree / held,
            "note": "slots held in one layer's pool after the run against the distinct "
                    "tokens of the beam tree (the same run on one-token blocks, which "
                    "have no tails and never copy)"},
        "cpu_baseline": None if oracle_in is None else cpu_baseline_beam(
            c, plens, oracle_in, choices[0], scale, args.seed),
    }


def cpu_baseline_beam(c, plens, h, pick0, scale, seed):
    """The float64 oracle on the host over the first beam step from the
    starting state (prompts stored and forked by the oracle's own allocator
    and cache writes, untimed): the selection (forks, frees), every beam's
    next slot and copy-on-write pairs, then for one layer the block copies,
    the new tokens' store and the attention of every beam.  The step's
    estimate adds the layer part once per layer."""
    import oracle.alloc as oa
    import oracle.decode as od
    R, W, L, bs, NB = c["requests"], c["width"], c["layers"], c["bs"], c["NB"]
    shape = (NB, c["Hkv"], bs, c["D"])
    kc = np.zeros(shape, dtype=h["pk"].dtype)
    vc = np.zeros(shape, dtype=h["pk"].dtype)
    alloc = oa.Allocator(NB, bs, init_order=np.random.default_rng(seed).permutation(NB))
    beams, nxt = [], R
    for r in range(R):
        n = int(plens[r])
        alloc.create(r)
        slots = [alloc.append(r)[0] for _ in range(n)]
        od.reshape_and_cache(h["pk"][:n], h["pk"][:n], kc, vc, slots, inplace=True)
        group = [r]
        for _ in range(W - 1):
            alloc.fork(r, nxt)
            group.append(nxt)
            nxt += 1
        beams.append(group)
    t0 = time.perf_counter()
    new = []
    for cur, pick in zip(beams, pick0):
        used, nb = set(), []
        for i in pick:                      # a beam chosen again is forked
            if i not in used:
                used.add(i)
                nb.append(cur[i])
            else:
                alloc.fork(cur[i], nxt)
                nb.append(nxt)
                nxt += 1
        for i, sid in enumerate(cur):       # a beam nobody chose is freed
            if i not in used:
                alloc.release(sid)
        new.append(nb)
    flat = [b for g in new for b in g]
    res = [alloc.append(b) for b in flat]
    t1 = time.perf_counter()
    od.copy_blocks([kc], [vc], [(x[1], x[2]) for x in res if x[1] >= 0], inplace=True)
    od.reshape_and_cache(h["nk"], h["nk"], kc, vc, [x[0] for x in res], inplace=True)
    MB = max(len(alloc.table(b)) for b in flat)
    tables, lens = alloc.build_batch(flat, MB)
    od.paged_decode(h["q"], kc, vc, np.array(tables), np.array(lens), scale, c["dtype"])
    t2 = time.perf_counter()
    secs = (t1 - t0) + L * (t2 - t1)
    ctx = int(np.sum(np.asarray(lens, dtype=np.int64)))
    from paged_kv_cache_198_amd import synth
    logical = L * ctx * 2 * c["Hkv"] * c["D"] * synth.ELEM_BYTES[c["dtype"]]
    cores, blas = host_threads()
    return {"value": logical / secs / 1e9, "unit": "GB/s", "cores": blas, "kind": "oracle",
            "s_per_step_estimate": secs, "host_s": t1 - t0, "layer_s": t2 - t1,
            "host_cores": cores, "blas_threads": blas,
            "sample": f"the first beam step: selection and slots once, then layer 0 of {L} "
                      f"(copies, cache write, attention of {len(flat)} beams) timed once and "
                      f"counted {L} times; float64 numpy"}


def run_decode(args, pa, synth, torch):
    """One decode workload in this process: the fused step, the two-call
    step, optionally the read probes and the oracle baseline."""
    workload = args.workload or "llama13b"
    print(f"[bench] building workload {workload} bs={args.bs}", file=sys.stderr, flush=True)
    st = Step(pa, synth, torch, args.bs, args.seed, args.partition, workload)
    w = st.w
    oracle_step = None
    if not args.no_cpu_baseline:
        # the oracle's host inputs, copied before any GPU step writes the pools
        print("[bench] oracle inputs to the host", file=sys.stderr, flush=True)
        oracle_step = OracleStep(st, args.cpu_budget)
    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    # The two forms alternate over three rounds (each round: W warm-up
    # steps, then exactly K timed steps per form) and each form's median is
    # kept, so neither is always the one timed first after the set-up.
    runs = {False: [], True: []}
    for _ in range(3):
        for fused in (False, True):
            runs[fused].append(st.run(args.steps, args.warmup, fused=fused))
    med = lambda rs: sorted(rs)[len(rs) // 2]
    two_ms, wall_two = med(runs[False])
    fused_ms, wall_fused = med(runs[True])
    kern_ms = st.kernel_time(args.steps, args.warmup)
    # the step is quoted on whichever form is faster on this workload
    fused_wins = fused_ms < two_ms
    step_ms = fused_ms if fused_wins else two_ms
    wall = wall_fused if fused_wins else wall_two
    lens_h = st.lens.cpu().numpy().astype(np.int64)
    blocks = (lens_h + w.bs - 1) // w.bs
    # closed form: with residues spread evenly, a sequence's last block
    # leaves (bs - 1) / 2 slots empty on average
    mod_w = len(lens_h) * (w.bs - 1) / 2
    # roofline: algorithmic K/V bytes over the attention launch's own
    # average duration (events right around it on the launch stream)
    achieved = st.kv_bytes / (kern_ms * 1e-3) / 1e9
    step_gbs = st.kv_bytes / (step_ms * 1e-3) / 1e9
    headline = workload == "llama13b"
    line = {
        "metric": "decode-attention KV GB/s (frac of MI355X HBM peak) + us/step, "
                  + ("13B-shaped batch" if headline else f"{workload} batch"),
        "value": step_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "us_per_step": step_ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, " + (
            "lognormal" if synth.CONFIGS[workload]["lengths"][0] == "lognormal" else "uniform")
            + " context lengths)",
        "config": {
            "workload": describe(workload, w),
            "S": w.S, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "block_size": w.bs,
            "tokens": int(np.sum(w.context_lens)), "kv_bytes": st.kv_bytes,
            "partition_tokens": st.part, "seed": args.seed,
        },
        "frac_hbm_peak_step": step_gbs / HBM_PEAK_GBS,
        "step": "fused" if fused_wins else "two_call",
        "two_call_step": {"us_per_step": two_ms * 1e3,
                          "GBs": st.kv_bytes / (two_ms * 1e-3) / 1e9,
                          "rounds_us": [r[0] * 1e3 for r in runs[False]],
                          "note": "pa_reshape_and_cache + pa_decode_attention as two launches"},
        "fused_step": {"us_per_step": fused_ms * 1e3,
                       "GBs": st.kv_bytes / (fused_ms * 1e-3) / 1e9,
                       "rounds_us": [r[0] * 1e3 for r in runs[True]],
                       "note": "pa_decode_step: the cache write folded into the attention launch"},
        "tail_waste": float((blocks * w.bs - lens_h).sum() / (blocks * w.bs).sum()),
        "tail_waste_model": float(mod_w / (lens_h.sum() + mod_w)),
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_bytes() if (headline and args.bs == 16) else None,
            "kernel": kernel_name(st),
            "kernel_us": kern_ms * 1e3,
            "algorithmic_bytes_per_launch": st.kv_bytes,
        },
        "wall_s_timed": wall,
    }
    if not args.no_probe:
        line["hbm_probe"] = hbm_probe(torch)
        # the practical ceiling: a plain streaming read of the decode's byte
        # count, and of 4 GiB
        alg = line["roofline"]["algorithmic_bytes_per_launch"]
        # One, two and sixteen 256-thread workgroups per CU: a light load
        # (about 32 KB in flight per CU) reads fastest on this part; the
        # best of the three is the practical ceiling.
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        grids = sorted({cus, 2 * cus, min(16 * cus, 4096)})
        same = read_probe(pa, torch, int(alg) // 16 * 16, grids)
        big = read_probe(pa, torch, 4 << 30, grids)
        line["hbm_probe"]["pa_read_probe_GBs"] = {
            "same_bytes": max(same.values()), "4GiB": max(big.values()),
            "by_workgroups": {str(g): {"same_bytes": same[g], "4GiB": big[g]} for g in grids}}
        line["roofline"]["frac_of_read_probe"] = line["roofline"]["achieved"] / max(same.values())
    if args.calibrate_copy:
        calibrate_copy(torch)
    if oracle_step is not None:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        line["cpu_baseline"] = oracle_step.time(gpu_out=st.out)
    else:
        line["cpu_baseline"] = None
    return line


# The default run's children: (key, arguments).  The headline comes first;
# the block-size sweep and the other workloads follow, one process each, so
# no measurement runs in a process that already holds another workload's
# device memory.
SWEEP_BS = (8, 16, 32, 64, 128)
CONFIG_RUNS = [
    ("tiny", ["--workload", "tiny", "--no-probe"]),
    ("llama7b", ["--workload", "llama7b", "--no-probe"]),
    ("shared_prefix_504", ["--workload", "shared_prefix", "--prompt-len", "504"]),
    ("shared_prefix_512", ["--workload", "shared_prefix", "--prompt-len", "512"]),
    ("long_gqa", ["--workload", "long_gqa", "--no-probe"]),
]


def decode_summary(r):
    """The per-workload record kept under ``configs`` / ``sweep``."""
    out = {"workload": r["config"]["workload"], "dtype": r["dtype"],
           "us_per_step": r["us_per_step"], "step": r["step"], "GBs": r["value"],
           "frac_hbm_peak_step": r["frac_hbm_peak_step"],
           "kernel": r["roofline"]["kernel"], "kernel_us": r["roofline"]["kernel_us"],
           "kernel_GBs": r["roofline"]["achieved"], "frac_hbm_peak": r["roofline"]["frac"],
           "kv_bytes": r["config"]["kv_bytes"],
           "partition_tokens": r["config"]["partition_tokens"],
           "two_call_us_per_step": r["two_call_step"]["us_per_step"],
           "fused_us_per_step": r["fused_step"]["us_per_step"],
           "tail_waste": r["tail_waste"], "tail_waste_model": r["tail_waste_model"]}
    if r.get("cpu_baseline") is not None:
        out["cpu_baseline"] = r["cpu_baseline"]
    return out


def shared_summary(r):
    c = r["config"]
    return {"workload": c["workload"], "dtype": r["dtype"],
            "plain": {"us_per_step": r["plain_fused_step"]["us"],
                      "logical_GBs": r["plain_fused_step"]["logical_GBs"],
                      "kernel": r["plain_fused_step"]["kernel"]},
            "cascade": {"us_per_step": r["us_per_step"], "logical_GBs": r["value"],
                        "read_GBs": r["roofline"]["achieved"],
                        "frac_hbm_peak_read": r["roofline"]["frac"],
                        "kernel": "pa::decode_gqa_mfma_kernel over work items + reduce_kernel "
                                  "(pa_decode_cascade, fused cache write)"},
            "kv_bytes": {"logical": c["logical_kv_bytes"], "read_by_cascade": c["cascade_kv_bytes"],
                         "unique": c["unique_kv_bytes"]},
            "sharing": r["sharing"], "cow_copy": r.get("cow_copy"),
            "cpu_baseline": r["cpu_baseline"]}


def prefill_summary(r):
    """The prefill record kept in the default line."""
    return {"workload": r["config"]["workload"], "dtype": r["dtype"],
            "us_per_step": r["us_per_step"], "prompt_tokens_per_s": r["value"],
            "kernel": r["roofline"]["kernel"], "kernel_us": r["roofline"]["kernel_us"],
            "TFLOPs": r["roofline"]["achieved"], "frac_bf16_mfma_peak": r["roofline"]["frac"],
            "back_to_back_us": r["back_to_back_us"], "flops_per_step": r["config"]["flops_per_step"],
            "cpu_baseline": r["cpu_baseline"]}


def launcher(args):
    """The default run.  This process never touches the GPU: every
    measurement runs in a child process, one after another.  A child that
    fails stops the run (nothing more is started), and the line printed so
    far carries the error."""
    base = [sys.executable, os.path.abspath(__file__), "--steps", str(args.steps),
            "--warmup", str(args.warmup), "--seed", str(args.seed),
            "--cpu-budget", str(args.cpu_budget)]
    if args.no_cpu_baseline:
        base.append("--no-cpu-baseline")

    def child(extra):
        print(f"[bench] child: {' '.join(extra)}", file=sys.stderr, flush=True)
        try:
            r = subprocess.run(base + extra, stdout=subprocess.PIPE, text=True, timeout=300)
        except subprocess.TimeoutExpired:
            return None, f"child {' '.join(extra)} ran past 300 s and was stopped"
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            return None, f"child {' '.join(extra)} exited with {r.returncode}"
        return json.loads(lines[-1]), None

    extra = ["--workload", "llama13b", "--bs", str(args.bs)]
    if args.no_probe:
        extra.append("--no-probe")
    if args.calibrate_copy:
        extra.append("--calibrate-copy")
    line, err = child(extra)
    if err:
        print(json.dumps({"error": err}), flush=True)
        sys.exit(1)
    for k in ("tail_waste", "tail_waste_model"):
        line.pop(k, None)
    line["sweep"], line["configs"] = {}, {}
    if not args.no_sweep:
        runs = [(f"bs{bs}", ["--workload", "llama13b", "--bs", str(bs), "--no-probe",
                             "--no-cpu-baseline"]) for bs in SWEEP_BS if bs != args.bs]
        runs += CONFIG_RUNS
        for key, extra in runs:
            r, err = child(extra)
            if err:
                line["error"] = err
                print(json.dumps(line), flush=True)
                sys.exit(1)
            if key.startswith("bs"):
                line["sweep"][key] = decode_summary(r)
            elif key.startswith("shared_prefix"):
                line["configs"][key] = shared_summary(r)
            else:
                line["configs"][key] = decode_summary(r)
        line["sweep"]["note"] = ("each block size in a process of its own, after the "
                                 f"headline (bs {args.bs})")
        # paged prefill of a 13B-shaped prompt batch (causal attention over
        # the blocks the prompts were written to)
        r, err = child(["--workload", "prefill"])
        if err:
            line["error"] = err
            print(json.dumps(line), flush=True)
            sys.exit(1)
        line["prefill"] = prefill_summary(r)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU benchmark: the decode path is not sharded over GPUs; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload is None:
        launcher(args)
        return
    import torch
    import paged_kv_cache_198_amd as pa
    from paged_kv_cache_198_amd import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    pa.lib()
    if args.workload == "prefill":
        print("[bench] prefill", file=sys.stderr, flush=True)
        print(json.dumps(run_prefill(args, pa, synth, torch)), flush=True)
        return
    if args.workload == "beam":
        print("[bench] beam search", file=sys.stderr, flush=True)
        print(json.dumps(run_beam(args, pa, synth, torch)), flush=True)
        return
    if args.workload in ("shared_prefix", "system_prompt"):
        print(f"[bench] building {args.workload} state", file=sys.stderr, flush=True)
        print(json.dumps(run_shared_prefix(args, pa, synth, torch)), flush=True)
        return
    print(json.dumps(run_decode(args, pa, synth, torch)), flush=True)


if __name__ == "__main__":
    main()
