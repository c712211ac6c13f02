"""Paged decode (and prefill) benchmark on one MI355X.

A step is one pass of the decode hot path over one batch: write the batch's
new-token K/V rows into their cache slots (pa_write_kv), then decode attention
for every sequence over its paged cache (pa_decode: partition kernel plus the
log-sum-exp merge).  Default workload: Llama-3-8B-shaped GQA, bf16, 256
sequences, 32 query / 8 KV heads, head_dim 128, block_size 16, context lengths
lognormal (median 1024, sigma 0.8) clipped to [16, 8192], blocks placed by a
seeded random permutation.  The pool holds `--layers` copies of the batch
(one per layer slot) and consecutive steps use consecutive layers, so a step
never finds the previous step's K/V in the 256 MB Infinity Cache.

Prints one JSON line.  value = KV-read GB/s = algorithmic KV bytes of one step
(valid tokens only: sum(ctx) * 2 * H_kv * D * 2 B) / wall time per step.

`--workload prefill_llama3_8b | chunked_llama3_8b | prefill_tiny` times the
prefill path instead: a step writes every sequence's new tokens (one batched
pa_write_kv) and runs pa_prefill over them; value = causal-attention TFLOP/s.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode KV-read GB/s (% of HBM peak) + seqs/s, Llama-3-8B-shaped GQA b=256"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["tiny", "opt13b", "llama3_8b", "long_ctx", "shared", "shared_cow",
                             "prefill_tiny", "prefill_llama3_8b", "chunked_llama3_8b", "prefix_cache",
                             "swap", "probe"])
    ap.add_argument("--contiguous", action="store_true",
                    help="place every sequence's blocks side by side in logical order (a "
                         "contiguous-cache control for the same kernel)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="decode workloads: a step is pa_write_kv then pa_decode (two calls) instead of "
                         "pa_decode_step (one call, the write beside the plan)")
    ap.add_argument("--share-plan", choices=["host", "device"], default="host",
                    help="shared-prefix workloads: the sharing groups come from the block manager on the "
                         "host (pa_batch_share_plan, pa_decode_step_shared) or are found by the device plan")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--partition-tokens", type=int, default=-1,
                    help="-1: the workload's own setting (0 = library default)")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0,
                    help="wall-clock budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-blocks", type=int, default=0,
                    help="after timing, copy this many whole blocks with pa_copy_blocks (a copy "
                         "of known size for scaling hardware byte counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_sha256(paths) -> str:
    """SHA-256 over the listed source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def run_steps(step, first, steps, stream):
    """Runs step(k) for k = first ... first+steps-1 back to back, as a serving
    loop would: wall clock and one stream event on each side of the whole loop,
    nothing recorded between steps.  Returns (wall ms per step, event ms per
    step)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(steps):
        step(first + k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, e0.elapsed_time(e1) / steps


def call_times(step, first, steps, stream):
    """Per-call durations (ms) of the hot-path call inside step: the same steps
    again, step(k, ev) recording ev[0] just before that call and ev[1] just after
    it on the stream the call launches on.  An event record leaves the stream
    idle for a few microseconds, so this pass is kept apart from run_steps."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        step(first + k, evs[k])
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def copy_calibration(pool, w, layers, blocks):
    """Copies `blocks` whole blocks (every layer) with pa_copy_blocks after the
    timed work: a copy of known size (returned, read and written once each)
    for scaling the FETCH_SIZE / WRITE_SIZE counters of the same run."""
    import torch
    import paged_kv_cache_337_amd as pa
    n = min(blocks, w.num_blocks // 2)
    pairs = torch.stack([torch.arange(n), torch.arange(n) + n], dim=1).to(torch.int32).cuda()
    pool.copy_blocks(pairs)
    torch.cuda.synchronize()
    nbytes = n * layers * 2 * w.num_kv_heads * w.block_size * w.head_dim * pa.ELEM_BYTES[w.dtype]
    log(f"[bench] copy calibration: {n} blocks, {nbytes} bytes read and {nbytes} written")
    return nbytes


# committed rocprofv3 counter records of the decode workloads
PROFILE_RECORDS = {"llama3_8b": "decode_llama3_8b_b256", "opt13b": "decode_opt13b_b64",
                   "long_ctx": "decode_long_ctx_b8", "shared": "decode_shared_b64",
                   "prefill_llama3_8b": "prefill_llama3_8b", "chunked_llama3_8b": "prefill_chunked_llama3_8b"}


def counter_traffic(record: str, workload: str, call: str | None = None):
    """HBM bytes per call from a committed rocprofv3 counter record
    (profiles/<record>.traffic.json: FETCH_SIZE + WRITE_SIZE, scaled by a copy
    of known size), or None when the record is for another workload or call
    (when one is named),
    or any of the kernels' sources changed since it was taken."""
    rec = os.path.join(ROOT, "profiles", record + ".traffic.json")
    if not os.path.exists(rec):
        return None
    with open(rec) as f:
        r = json.load(f)
    if (r.get("workload") != workload or (call is not None and r.get("call") != call)
            or r.get("sources_sha256") != sources_sha256(r["kernel_sources"])):
        return None
    return int(r["traffic_bytes_per_call"])


def cpu_baseline(w, budget_s, tables, ctx):
    """Time the CPU oracle as it stands (gather through the block table, then
    float64 two-pass softmax) on the first sequences of the same batch, until
    the wall-clock budget is spent."""
    from oracle import attention as A
    from oracle import layout as LY
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    g = LY.Geometry(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    pool = np.zeros(g.num_elements, dtype=np.uint16 if w.dtype != "f32" else np.float32)
    done, kv_bytes, t_total = 0, 0, 0.0
    eb = 4 if w.dtype == "f32" else 2
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        LY.scatter(pool, g, 0, tables[i], K, V)  # input staging, not timed
        t0 = time.perf_counter()
        A.paged_decode(pool, g, 0, w.q, tables, ctx, w.scale, seqs=[i])
        t_total += time.perf_counter() - t0
        done += 1
        kv_bytes += int(ctx[i]) * 2 * w.num_kv_heads * w.head_dim * eb
        if t_total >= budget_s:
            break
    return {
        "value": round(kv_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "seqs_per_s": round(done / t_total, 3),
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"first {done} of {w.num_seqs} sequences of the same batch "
                  f"({int(ctx[:done].sum())} tokens), {t_total:.1f} s of oracle time",
    }


def prefill_flops(w) -> int:
    """Causal attention flops of a prefill batch: per new token and query
    head, 2*D for q.k and 2*D for p.v per key it attends to."""
    total = 0
    for c, n in zip(w.context_lens.astype(np.int64), w.query_lens.astype(np.int64)):
        keys = n * (c - n) + n * (n + 1) // 2  # sum over new tokens of (position + 1)
        total += int(keys)
    return 4 * w.head_dim * w.num_q_heads * total


def cpu_baseline_prefill(w, budget_s):
    """The oracle's causal prefill on the new tokens of the first sequences,
    one token at a time, until the budget is spent."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    qs = w.query_start
    flops, rows, t_total = 0, 0, 0.0
    for i in range(w.num_seqs):
        K, V = (A.to_f64(x, w.dtype) for x in w.seq_kv(i))
        q = A.to_f64(w.q[qs[i]:qs[i + 1]], w.dtype)
        c, n = K.shape[0], q.shape[0]
        for k in range(n):
            t0 = time.perf_counter()
            A.prefill_one(q, K, V, w.scale, rows=[k])
            t_total += time.perf_counter() - t0
            flops += 4 * w.head_dim * w.num_q_heads * (c - n + k + 1)
            rows += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "tokens_per_s": round(rows / t_total, 2),
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"first {rows} new tokens of the same batch (sequence order), {t_total:.1f} s of oracle time",
    }


PREFILL_METRIC = "paged causal prefill attention TFLOP/s (% of bf16 MFMA peak), Llama-3-8B-shaped GQA"
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}


def main_prefill(args):
    """A step: one batched pa_write_kv of every sequence's new tokens, then
    pa_prefill of those tokens over their cached contexts."""
    import torch
    import paged_kv_cache_337_amd as pa
    import workloads as W
    from paged_kv_cache_337_amd import staging as U

    w = W.PREFILL_WORKLOADS[args.workload]()
    eb = pa.ELEM_BYTES[w.dtype]
    L = max(1, args.layers)
    log(f"[bench] workload={w.name} S={w.num_seqs} context tokens={w.total_tokens} "
        f"new tokens={int(w.query_lens.sum())} blocks={w.num_blocks} layers={L}")
    t0 = time.time()
    pool = U.make_pool(w, layers=L)
    for layer in range(L):
        U.fill_pool(pool, w, layer=layer)
    log(f"[bench] pool filled ({pool.nbytes / 1e9:.2f} GB) in {time.time() - t0:.1f} s")
    qs_h = w.query_start
    first = (w.context_lens - w.query_lens).astype(np.int32)
    slots_new = pa.slots_for_positions(w.block_tables, w.block_size, first, w.query_lens)
    kn = np.concatenate([w.seq_kv(i)[0][first[i]:] for i in range(w.num_seqs)])
    vn = np.concatenate([w.seq_kv(i)[1][first[i]:] for i in range(w.num_seqs)])
    k_new, v_new = U.dev_tensor(kn, w.dtype), U.dev_tensor(vn, w.dtype)
    slot_new = torch.from_numpy(slots_new).cuda()
    q, qs, tables, ctx = U.prefill_inputs(w)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    max_q, max_ctx = w.max_query_len, w.max_context_len

    def step(k, ev=None):
        layer = k % L
        pool.write_kv(layer, k_new, v_new, slot_new)
        if ev is not None:
            ev[0].record(stream)
        pool.prefill(layer, q, qs, max_q, tables, ctx, max_ctx, w.scale, out=out)
        if ev is not None:
            ev[1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite prefill output")
    ms_per_step, _ = run_steps(step, args.warmup, args.steps, stream)
    pf_ms = float(np.mean(call_times(step, args.warmup + args.steps, args.steps, stream)))
    flops = prefill_flops(w)
    ntok = int(qs_h[-1])
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (pf_ms * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: paged causal prefill, {w.num_seqs} seqs, {ntok} new tokens over "
                        f"{w.total_tokens} context tokens, {w.num_q_heads}q/{w.num_kv_heads}kv heads, "
                        f"head_dim {w.head_dim}, block_size {w.block_size}",
            "batch": w.num_seqs, "new_tokens": ntok, "total_context_tokens": w.total_tokens,
            "max_query_len": max_q, "max_context_len": max_ctx, "layer_slots_rotated": L,
            "step": "pa_write_kv (all new tokens) + pa_prefill",
        },
        "tokens_per_s": round(ntok / (ms_per_step * 1e-3), 1),
        "flops_per_step": flops,
        "roofline": {
            "bound": "mfma",
            "kernel": ("pa_prefill (prefill_lds_kernel)" if eb == 2 else "pa_prefill (prefill_kernel)"),
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": (counter_traffic(PROFILE_RECORDS[w.name], w.name)
                        if w.name in PROFILE_RECORDS and L == 4 else None),
            "traffic_unit": "bytes per launch (HBM)",
            "alg_flops_per_launch": flops,
            "kv_bytes_per_launch": w.total_tokens * 2 * w.num_kv_heads * w.head_dim * eb,
            "avg_launch_ms": round(pf_ms, 5),
        },
    }
    if args.copy_calib_blocks > 0:
        res["copy_calibration_bytes"] = copy_calibration(pool, w, L, args.copy_calib_blocks)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


PREFIX_METRIC = "shared-system-prompt admission: requests/s with automatic prefix caching (write + prefill)"


def main_prefix(args):
    """64 Llama-3-8B-shaped requests share a 1024-token system prompt (each
    adds a 64..256-token question).  With prefix caching the prompt's whole
    blocks are found in the cache, so a step writes and prefills only the
    rest; without it a step writes and prefills every token.  The prompt is
    kept cached by a pinned sequence, as a served system prompt would be."""
    import torch
    import paged_kv_cache_337_amd as pa
    import workloads as W
    from paged_kv_cache_337_amd import staging as U

    w = W.prefix_cache()
    R, bs = w.num_requests, w.block_size
    reqs = list(range(R))
    lens = [len(w.request_ids(r)) for r in reqs]
    total = sum(lens)
    N = sum(-(-n // bs) for n in lens) * 2 + 64
    pool = pa.Pool(1, N, bs, w.num_kv_heads, w.head_dim, w.dtype)
    U.poison(pool)
    log(f"[bench] prefix_cache: {R} requests, prompt {len(w.prompt_ids)}, {total} tokens, pool {N} blocks")

    # without the cache: every token is appended, written and prefilled
    plain = U.run_prefix_requests(pool, w, reqs)
    assert all(nc == 0 for _, nc in plain)
    in_plain = U.prefix_prefill_inputs(pool, w, plain, reqs)
    k_all = U.dev_tensor(np.concatenate([w.request_kv(r)[0] for r in reqs]), w.dtype)
    v_all = U.dev_tensor(np.concatenate([w.request_kv(r)[1] for r in reqs]), w.dtype)
    slots_plain = torch.from_numpy(pa.slots_for_positions(
        pool.batch_tables([s for s, _ in plain], max(-(-n // bs) for n in lens))[0], bs,
        np.zeros(R, dtype=np.int32), np.array(lens, dtype=np.int32))).cuda()

    # with the cache: a pinned sequence holds the prompt; requests are admitted
    pool.enable_prefix_cache(True)
    pin = pool.seq_create()
    pslots, _, _ = pool.seq_append_tokens(pin, w.prompt_ids)
    pk, pv = w.prompt_kv()
    pool.write_kv(0, U.dev_tensor(pk, w.dtype), U.dev_tensor(pv, w.dtype), torch.from_numpy(pslots).cuda())
    cached = U.run_prefix_requests(pool, w, reqs)
    n_cached = sum(nc for _, nc in cached)
    in_cached = U.prefix_prefill_inputs(pool, w, cached, reqs)
    kc = U.dev_tensor(np.concatenate([w.request_kv(r)[0][nc:] for r, (_, nc) in zip(reqs, cached)]), w.dtype)
    vc = U.dev_tensor(np.concatenate([w.request_kv(r)[1][nc:] for r, (_, nc) in zip(reqs, cached)]), w.dtype)
    slc = []
    for r, (s, nc) in zip(reqs, cached):
        tbl = np.array(pool.seq_block_table(s)[0], dtype=np.int32)
        pos = np.arange(nc, lens[r])
        slc.append(tbl[pos // bs] * bs + pos % bs)
    slots_cached = torch.from_numpy(np.concatenate(slc).astype(np.int32)).cuda()
    stream = torch.cuda.current_stream()

    def timed(kk, vv, slots, inp, steps, warmup):
        q, qs, t, c, mq, mc = inp
        out = torch.empty_like(q)
        for _ in range(warmup):
            pool.write_kv(0, kk, vv, slots)
            pool.prefill(0, q, qs, mq, t, c, mc, w.scale, out=out)
        torch.cuda.synchronize()
        def step(_k, e=None):
            pool.write_kv(0, kk, vv, slots)
            if e is not None:
                e[0].record(stream)
            pool.prefill(0, q, qs, mq, t, c, mc, w.scale, out=out)
            if e is not None:
                e[1].record(stream)

        wall_ms, _ = run_steps(step, 0, steps, stream)
        pf_ms = float(np.mean(call_times(step, 0, steps, stream)))
        if not torch.isfinite(out.float()).all():
            raise RuntimeError("non-finite prefill output")
        return wall_ms, pf_ms

    ms_c, pf_c = timed(kc, vc, slots_cached, in_cached, args.steps, args.warmup)
    ms_p, pf_p = timed(k_all, v_all, slots_plain, in_plain, args.steps, args.warmup)

    def flops(admitted):
        tot = 0
        for r, (_, nc) in zip(reqs, admitted):
            n, c = lens[r] - nc, lens[r]
            tot += n * (c - n) + n * (n + 1) // 2
        return 4 * w.head_dim * w.num_q_heads * tot

    # block-manager cost alone (host-only pool, no device work): one
    # pa_seq_append_tokens per request, without and with the cache; the
    # median of three passes, with Python's cyclic collector paused (a full
    # collection of the interpreter's heap takes tens of milliseconds)
    ids_all = [w.request_ids(r) for r in reqs]
    plain_t, cached_t = [], []
    for _ in range(3):
        hp = pa.Pool(1, N, bs, w.num_kv_heads, w.head_dim, w.dtype, device=None)
        gc.disable()
        try:
            t0 = time.perf_counter()
            hs = [hp.seq_create() for _ in reqs]
            for sq, ids in zip(hs, ids_all):
                hp.seq_append_tokens(sq, ids)
            plain_t.append(time.perf_counter() - t0)
            for sq in hs:
                hp.seq_release(sq)
            hp.enable_prefix_cache(True)
            hp.seq_append_tokens(hp.seq_create(), w.prompt_ids)
            t0 = time.perf_counter()
            hs = [hp.seq_create() for _ in reqs]
            for sq, ids in zip(hs, ids_all):
                hp.seq_append_tokens(sq, ids)
            cached_t.append(time.perf_counter() - t0)
        finally:
            gc.enable()
        del hp
    host_plain = float(np.median(plain_t))
    host_cached = float(np.median(cached_t))

    f_c = flops(cached)
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    achieved = f_c / (pf_c * 1e-3) / 1e12
    res = {
        "metric": PREFIX_METRIC,
        "value": round(R / (ms_c * 1e-3), 1),
        "unit": "requests/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_c, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"prefix_cache: {R} requests sharing a {len(w.prompt_ids)}-token system prompt, "
                        f"questions 64-256 tokens ({total} tokens), {w.num_q_heads}q/{w.num_kv_heads}kv heads, "
                        f"head_dim {w.head_dim}, block_size {bs}, one layer",
            "step": "pa_write_kv (tokens the cache did not serve) + pa_prefill (those tokens)",
        },
        "tokens_served_from_cache": n_cached,
        "tokens_written_and_prefilled": total - n_cached,
        "without_cache": {"requests_per_s": round(R / (ms_p * 1e-3), 1), "ms_per_step": round(ms_p, 5),
                          "prefill_ms": round(pf_p, 5), "tflops": round(flops(plain) / (pf_p * 1e-3) / 1e12, 2)},
        "speedup_vs_no_cache": round(ms_p / ms_c, 3),
        "host_block_manager_us_per_request": {
            "cached": round(host_cached * 1e6 / R, 2), "no_cache": round(host_plain * 1e6 / R, 2),
            "note": "pa_seq_create + pa_seq_append_tokens through ctypes, host-only pool; median of 3 passes, "
                    "Python garbage collection paused"},
        "prefix_cache_stats": pool.prefix_cache_stats(),
        "roofline": {
            "bound": "mfma",
            "kernel": "pa_prefill (prefill_lds_kernel) over the uncached tokens",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "alg_flops_per_launch": f_c,
            "avg_launch_ms": round(pf_c, 5),
        },
    }
    print(json.dumps(res), flush=True)


SWAP_METRIC = "swap of whole sequences between the paged pool and pinned host memory, GB/s per direction"


def main_swap(args):
    """Every sequence of the Llama-3-8B-shaped decode batch (256 sequences,
    1.5 GB of K/V in one layer) is swapped out to pinned host memory and back
    in: block-manager calls, then one pa_swap_blocks launch per direction.  The
    link's reference rate is a PyTorch copy of the same number of bytes between
    a device tensor and a pinned host tensor (DMA engines)."""
    import torch
    import paged_kv_cache_337_amd as pa
    import workloads as W
    from paged_kv_cache_337_amd import staging as U

    w = W.llama3_8b()
    S, bs = w.num_seqs, w.block_size
    pool = pa.Pool(1, w.num_blocks, bs, w.num_kv_heads, w.head_dim, w.dtype)
    U.poison(pool)
    seqs = [pool.seq_create() for _ in range(S)]
    for s, c in zip(seqs, w.context_lens):
        pool.seq_append(s, int(c))
    tables, ctx = pool.batch_tables(seqs, w.max_blocks_per_seq)
    U.fill_pool(pool, w, tables=tables)
    nblk = w.num_blocks
    pool.host_tier_init(nblk)
    hbb = pool.host_block_bytes
    host = torch.empty(nblk * hbb, dtype=torch.uint8, pin_memory=True)
    moved = nblk * hbb
    log(f"[bench] swap: {S} sequences, {nblk} blocks, {moved / 1e9:.2f} GB each way")
    stream = torch.cuda.current_stream()
    out_ms, in_ms, host_us = [], [], []
    for _ in range(args.warmup + args.steps):
        t0 = time.perf_counter()
        pairs = [p for s in seqs for p in pool.seq_swap_out(s)]
        host_us.append((time.perf_counter() - t0) * 1e6 / S)
        pt = torch.tensor(pairs, dtype=torch.int32).cuda()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pool.swap_blocks(pt, host, 0)
        e[1].record(stream)
        pairs = [p for s in seqs for p in pool.seq_swap_in(s)]
        pt = torch.tensor(pairs, dtype=torch.int32).cuda()
        e[2].record(stream)
        pool.swap_blocks(pt, host, 1)
        e[3].record(stream)
        torch.cuda.synchronize()
        out_ms.append(e[0].elapsed_time(e[1]))
        in_ms.append(e[2].elapsed_time(e[3]))
    out_ms, in_ms = out_ms[args.warmup:], in_ms[args.warmup:]
    # parity spot check: decode after the round trips equals decode before
    q, t, c = U.device_inputs(w, tables=np.asarray(pool.batch_tables(seqs, w.max_blocks_per_seq)[0]), ctx=ctx)
    out = pool.decode(0, q, t, c, w.max_context_len, w.scale, 0)
    torch.cuda.synchronize()
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite decode after swap")
    # reference: DMA copies of the same bytes
    dev = torch.empty(moved, dtype=torch.uint8, device="cuda")
    ref = []
    for direction in (0, 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for k in range(2):
            ev[0].record(stream)
            if direction == 0:
                host.copy_(dev, non_blocking=True)
            else:
                dev.copy_(host, non_blocking=True)
            ev[1].record(stream)
            torch.cuda.synchronize()
        ref.append(moved / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9)
    gb_out = moved / (float(np.mean(out_ms)) * 1e-3) / 1e9
    gb_in = moved / (float(np.mean(in_ms)) * 1e-3) / 1e9
    res = {
        "metric": SWAP_METRIC,
        "value": round(min(gb_out, gb_in), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(out_ms)) + float(np.mean(in_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"swap: llama3_8b batch, {S} sequences, {nblk} blocks of {hbb} B "
                               f"({moved / 1e9:.2f} GB) out to pinned host memory and back in",
                   "step": "pa_seq_swap_out x S + pa_swap_blocks(out), pa_seq_swap_in x S + pa_swap_blocks(in)"},
        "swap_out_gbs": round(gb_out, 2),
        "swap_in_gbs": round(gb_in, 2),
        "dma_copy_gbs": {"device_to_host": round(ref[0], 2), "host_to_device": round(ref[1], 2)},
        "host_block_manager_us_per_sequence": round(float(np.mean(host_us[args.warmup:])), 2),
        "roofline": {
            "bound": "host-link",
            "kernel": "swap_blocks_kernel (one launch per direction)",
            "achieved": round(min(gb_out, gb_in), 2),
            "peak": round(min(ref), 2),
            "unit": "GB/s",
            "frac": round(min(gb_out, gb_in) / min(ref), 4),
            "traffic": None,
            "note": "peak = the DMA-engine copy rate of the same bytes measured in this run",
        },
    }
    print(json.dumps(res), flush=True)


PROBE_FORMS = {0: "global_load_dwordx4 nt", 1: "global_load_dwordx4", 2: "buffer_load_dwordx4 nt",
               3: "global_load_lds_dwordx4", 4: "global_load_lds_dwordx4 nt"}


def main_probe(args):
    """HBM read rate of the decode kernel's access pattern (pa_probe_read_chunks:
    whole 8 KiB chunks, 16 bytes per lane per load, no arithmetic) over a 6 GiB
    buffer: by chunk order (random 8 KiB chunks -- one (block, kv head) region
    of the pool --, random runs of 4, 8 and 32 chunks, the identity order) with
    the decode kernel's loads, then random 8 KiB chunks with every load form
    of the probe, workgroups per CU and chunks in flight.  It bounds what any
    block placement, and any of these load forms, could gain."""
    import torch
    import paged_kv_cache_337_amd as pa
    nbytes = 6 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    nchunks = nbytes // 8192
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)

    def runs(g):
        starts = rng.permutation(nchunks // g)
        return (starts[:, None] * g + np.arange(g)[None, :]).reshape(-1).astype(np.int32)

    orders = {"random_8KiB": rng.permutation(nchunks).astype(np.int32), "random_32KiB_runs": runs(4),
              "random_64KiB_runs": runs(8), "random_256KiB_runs": runs(32),
              "identity": np.arange(nchunks, dtype=np.int32)}
    stream = torch.cuda.current_stream()

    def rate(od, form=0, wg=2, infl=2):
        def step(_k, ev):
            ev[0].record(stream)
            pa.probe_read_chunks(buf, od, sink, load_form=form, wg_per_cu=wg, in_flight=infl)
            ev[1].record(stream)

        ms = call_times(step, 0, 1 + max(args.steps // 20, 3), stream)
        return round(nbytes / (float(np.median(ms[1:])) * 1e-3) / 1e9, 1)  # first call warms up

    rates = {}
    for name, order in orders.items():
        rates[name] = rate(torch.from_numpy(order).cuda())
        log(f"[probe] order {name}: {rates[name]} GB/s")
    rnd = torch.from_numpy(orders["random_8KiB"]).cuda()
    forms = []
    for form, fname in PROBE_FORMS.items():
        for wg in (1, 2, 3):
            for infl in ((1, 2) if form >= 3 else (1, 2, 4)):
                r = rate(rnd, form, wg, infl)
                forms.append({"load_form": fname, "wg_per_cu": wg, "chunks_in_flight": infl, "gbs": r})
                log(f"[probe] {fname} wg/CU {wg} in flight {infl}: {r} GB/s")
    best = max(forms, key=lambda f: f["gbs"])
    print(json.dumps({"metric": "HBM read probe GB/s by chunk contiguity and load form (pa_probe_read_chunks, 6 GiB)",
                      "value": rates["random_8KiB"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                      "data": "synthetic", "rates": rates, "best_random_8KiB": best, "load_forms": forms,
                      "peak": HBM_PEAK_GBS}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this library runs on a single GPU; use --gpus 1"}))
        sys.exit(2)
    if args.workload.startswith(("prefill", "chunked")):
        return main_prefill(args)
    if args.workload == "prefix_cache":
        return main_prefix(args)
    if args.workload == "swap":
        return main_swap(args)
    if args.workload == "probe":
        return main_probe(args)

    import torch
    import paged_kv_cache_337_amd as pa
    import workloads as W
    from paged_kv_cache_337_amd import staging as U

    w = W.WORKLOADS[args.workload]()
    P = w.partition_tokens if args.partition_tokens < 0 else args.partition_tokens
    eb = pa.ELEM_BYTES[w.dtype]
    L = max(1, args.layers)
    log(f"[bench] workload={w.name} S={w.num_seqs} tokens={w.total_tokens} blocks={w.num_blocks} "
        f"layers={L} P={P}")

    t0 = time.time()
    shared = w.script is not None
    if shared:
        # prefix sharing through the block manager (fork, append, copy-on-write)
        pool = pa.Pool(L, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype,
                       free_order=w.script["free_order"])
        U.poison(pool)
        U.run_shared_script(pool, w, W.shared_prefix_kv, W.private_kv, layers=range(L))
        width = max(len(pool.seq_block_table(s)[0]) for s in range(w.num_seqs))
        host_tables, host_ctx = pool.batch_tables(list(range(w.num_seqs)), width)
    else:
        host_tables = U.contiguous_tables(w) if args.contiguous else w.block_tables
        host_ctx = w.context_lens
        pool = U.make_pool(w, layers=L)
        for layer in range(L):
            U.fill_pool(pool, w, layer=layer, tables=host_tables)
    log(f"[bench] pool filled ({pool.nbytes / 1e9:.2f} GB) in {time.time() - t0:.1f} s")

    # new-token inputs: each sequence's last position (its current token)
    last = host_ctx - 1
    kn = np.stack([w.seq_kv(i)[0][last[i]] for i in range(w.num_seqs)])
    vn = np.stack([w.seq_kv(i)[1][last[i]] for i in range(w.num_seqs)])
    slots_new = pa.slots_for_positions(host_tables, w.block_size, last, np.ones(w.num_seqs))
    k_new, v_new = U.dev_tensor(kn, w.dtype), U.dev_tensor(vn, w.dtype)
    slot_new = torch.from_numpy(slots_new).cuda()
    q, tables, ctx = U.device_inputs(w, tables=host_tables, ctx=host_ctx)
    out = torch.empty_like(q)
    ws_bytes = pool.workspace_bytes(w.num_seqs, w.num_q_heads, w.max_context_len, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    max_ctx = w.max_context_len

    fused = not args.separate_calls
    # Sharing groups from the block manager: made on the host beside the
    # tables (median of 5 host timings) and resident on the device like them.
    share_plan, host_plan_us = None, None
    if shared and args.share_plan == "host" and fused:
        rows = list(range(w.num_seqs))
        host_us = []
        for _ in range(5):
            t1 = time.perf_counter()
            plan_np = pool.batch_share_plan(rows, w.num_q_heads)
            host_us.append((time.perf_counter() - t1) * 1e6)
        host_plan_us = round(float(np.median(host_us)), 1)
        share_plan = torch.from_numpy(plan_np).cuda()
        log(f"[bench] host sharing plan: {int(plan_np[0])} subgroups in {host_plan_us} us")

    def step(k, ev=None):
        layer = k % L
        if fused:  # the new tokens' write beside the decode's plan, in one call
            if ev is not None:
                ev[0].record(stream)
            pool.decode_step(layer, k_new, v_new, slot_new, q, tables, ctx, max_ctx, w.scale, P, out=out,
                             workspace=ws, share_plan=share_plan)
            if ev is not None:
                ev[1].record(stream)
            return
        pool.write_kv(layer, k_new, v_new, slot_new)
        if ev is not None:
            ev[0].record(stream)
        pool.decode(layer, q, tables, ctx, max_ctx, w.scale, P, out=out, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite decode output")

    ms_per_step, ev_ms = run_steps(step, args.warmup, args.steps, stream)
    # The same steps again (continuing the layer rotation), timing each
    # pa_decode call on its stream.
    call_ms = call_times(step, args.warmup + args.steps, args.steps, stream)
    dec_ms = float(np.mean(call_ms))

    # Table-free comparison point on the same consecutive blocks: sequence
    # i's blocks are host_tables[i, 0] + k, read with no table at all.
    table_free = None
    if args.contiguous and not shared:
        first = torch.from_numpy(np.ascontiguousarray(host_tables[:, 0], dtype=np.int32)).cuda()

        def step_flat(k, ev=None):
            layer = k % L
            pool.write_kv(layer, k_new, v_new, slot_new)
            if ev is not None:
                ev[0].record(stream)
            pool.decode_contiguous(layer, q, first, ctx, max_ctx, w.scale, P, out=out, workspace=ws)
            if ev is not None:
                ev[1].record(stream)

        out_tab = out.clone()
        step_flat(0)
        torch.cuda.synchronize()
        step(0)
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), out_tab.view(torch.int16)):
            raise RuntimeError("table-free and table decode differ")
        flat_ms = call_times(step_flat, args.warmup + 2 * args.steps, args.steps, stream)
        flat_step_ms, _ = run_steps(step_flat, args.warmup + 3 * args.steps, args.steps, stream)
        table_free = {"kernel": "pa_decode_contiguous (no block table; consecutive blocks from each first block)",
                      "avg_launch_ms": round(float(np.mean(flat_ms)), 5),
                      "median_launch_ms": round(float(np.median(flat_ms)), 5),
                      "ms_per_step": round(flat_step_ms, 5)}

    # Warm calls: the same layer again and again (no rotation), so whatever
    # the Infinity Cache keeps between calls is found there.
    warm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in warm:
        a.record(stream)
        pool.decode(0, q, tables, ctx, max_ctx, w.scale, P, out=out, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    warm_ms = float(np.median([a.elapsed_time(b) for a, b in warm]))

    # Read probe over the pool buffer: every 8 KiB chunk once, in a seeded
    # random order (the decode kernel's access granularity, no arithmetic).
    nchunks = pool.nbytes // 8192
    order = torch.from_numpy(np.random.default_rng(0).permutation(nchunks).astype(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for a, b in pev:
        a.record(stream)
        pa.probe_read_chunks(pool.buf, order, sink)
        b.record(stream)
    torch.cuda.synchronize()
    probe_gbs = nchunks * 8192 / (float(np.median([a.elapsed_time(b) for a, b in pev[1:]])) * 1e-3) / 1e9
    tok_bytes = 2 * w.num_kv_heads * w.head_dim * eb
    kv_bytes = int(host_ctx.astype(np.int64).sum()) * tok_bytes
    nblk = int(sum(-(-int(c) // w.block_size) for c in host_ctx))
    # distinct cache slots the batch reads (below the logical count when blocks are shared)
    slots_read = set()
    for i in range(w.num_seqs):
        pos = np.arange(int(host_ctx[i]))
        slots_read.update((host_tables[i][pos // w.block_size].astype(np.int64) * w.block_size
                           + pos % w.block_size).tolist())
    unique_kv_bytes = len(slots_read) * tok_bytes
    qo_bytes = 2 * w.num_seqs * w.num_q_heads * w.head_dim * eb
    # The roofline counts each physical K/V byte once: a block that several
    # sequences share needs to be read from HBM only once (the logical bytes,
    # every sequence's whole context, are `value`'s measure and the
    # alg_bytes_logical field).  Without shared blocks the two are equal.
    other_bytes = qo_bytes + 4 * nblk + 4 * w.num_seqs
    if fused:  # the new tokens read from their rows and written to their slots, and the slots
        other_bytes += 2 * w.num_seqs * tok_bytes + 4 * w.num_seqs
    alg_bytes = unique_kv_bytes + other_bytes
    alg_bytes_logical = kv_bytes + other_bytes
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: paged decode layer, {w.num_seqs} seqs, {w.num_q_heads}q/{w.num_kv_heads}kv "
                        f"heads, head_dim {w.head_dim}, block_size {w.block_size}"
                        + (", contiguous block placement" if args.contiguous and not shared else ""),
            "batch": w.num_seqs, "total_context_tokens": w.total_tokens,
            "max_context_len": max_ctx,
            "partition_tokens": P if P else "automatic (at least 512, chosen on the device)",
            "layer_slots_rotated": L,
            "step": ("pa_decode_step (1 new token/seq written, then decode, one call)" if fused
                     else "pa_write_kv (1 new token/seq) + pa_decode")
                    if share_plan is None else
                    "pa_decode_step_shared (1 new token/seq written, then decode, one call; sharing groups "
                    "from the block manager)",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_logical": kv_bytes,
        "kv_bytes_unique": unique_kv_bytes,
        "unique_kv_gbs": round(unique_kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "seqs_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "event_ms_per_step": round(ev_ms, 5),
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_decode_step_shared call (prologue: the write beside the plan, which takes the "
                       "sharing groups from the host; decode kernel; merge kernel)" if share_plan is not None
                       else "pa_decode_step call (prologue: the write beside the plan; decode kernel; merge kernel)"
                       if fused else "pa_decode call (plan_kernel + decode kernel + merge_kernel)"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (counter_traffic(PROFILE_RECORDS[w.name], w.name,
                                        "pa_decode_step_shared" if share_plan is not None
                                        else "pa_decode_step" if fused else "pa_decode")
                        if w.name in PROFILE_RECORDS and P == w.partition_tokens and L == 4
                        and not args.contiguous else None),
            "alg_bytes_per_launch": alg_bytes,
            "alg_bytes_logical": alg_bytes_logical,
            "avg_launch_ms": round(dec_ms, 5),
            "median_launch_ms": round(float(np.median(call_ms)), 5),
            "warm_median_launch_ms": round(warm_ms, 5),
            "warm_achieved": round(alg_bytes / (warm_ms * 1e-3) / 1e9, 2),
            "probe_read_gbs": round(probe_gbs, 2),
            "frac_of_probe": round(achieved / probe_gbs, 4),
        },
    }
    if host_plan_us is not None:
        res["host_share_plan_us"] = host_plan_us
    if table_free is not None:
        table_free["achieved"] = round(alg_bytes / (table_free["avg_launch_ms"] * 1e-3) / 1e9, 2)
        table_free["kv_gbs_per_step"] = round(kv_bytes / (table_free["ms_per_step"] * 1e-3) / 1e9, 2)
        table_free["table_cost_pct"] = round(100 * (dec_ms / table_free["avg_launch_ms"] - 1), 2)
        res["table_free"] = table_free
    if args.copy_calib_blocks > 0:
        res["copy_calibration_bytes"] = copy_calibration(pool, w, L, args.copy_calib_blocks)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s, host_tables, host_ctx)
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                one = cpu_baseline(w, max(args.cpu_budget_s / 4, 1.0), host_tables, host_ctx)
            res["cpu_baseline"]["one_thread"] = {"value": one["value"], "sample": one["sample"]}
        except ImportError:  # pragma: no cover
            pass
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
