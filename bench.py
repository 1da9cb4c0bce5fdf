"""Benchmark of one MLA decode step on one MI355X.

A step is the whole decode hot path on one batch: write the newest latent row
of every sequence and absorb W_UK into the queries (mla_write_absorb, the
result of mla_write_cache then mla_absorb_q in one launch), then split-T
decode + LSE-merge combine with W_UV (mla_decode).  Default workload: DeepSeek-V3 attention shapes, B=64 sequences
of T=8192 cached tokens, H=128 heads, d_c=512, d_R=64, bf16, page size 64.

Prints one JSON line.  `value` is latent-cache GB/s of the step: the
algorithmic bytes (sum of sequence lengths x 576 values x 2 bytes) divided by
the step time; tokens/s (sequences decoded per second, per layer) rides along.

Besides the headline line's step, the JSON carries: the decode call alone at
every other decode workload (tiny fp32, V2-Lite, paged ragged), a measured
streaming-read ceiling of the GPU, the prefill and 8-bit-cache legs, the
float64 oracle timed on the host (cpu_baseline) and the run conditions.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload v3_decode]
       python bench.py --calibrate   (a 1 GiB device copy x 3, to scale the
                                      FETCH_SIZE / WRITE_SIZE counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_v3_counters.json")
DECODE_SRC = os.path.join(ROOT, "mla_latent_kv_22_amd", "csrc", "k_decode_mfma.hip")


def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def conditions():
    """Run conditions: host CPU, cores, ROCm / torch versions, GPU name, the
    code's identity (git SHA when the tree has one, else a hash of the
    sources)."""
    import platform
    import subprocess
    import torch
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        rocm = getattr(torch.version, "hip", None)
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except Exception:  # pragma: no cover
        sha = None
    h = hashlib.sha256()
    for sub in ("include", os.path.join("mla_latent_kv_22_amd", "csrc")):
        for dirpath, _, files in sorted(os.walk(os.path.join(ROOT, sub))):
            for fn in sorted(files):
                if fn.endswith((".h", ".hip")):
                    with open(os.path.join(dirpath, fn), "rb") as f:
                        h.update(fn.encode() + f.read())
    return {"gpu": torch.cuda.get_device_name(0), "cpu_model": cpu, "affinity_cpus": len(os.sched_getaffinity(0)),
            "rocm": rocm, "torch": torch.__version__, "python": platform.python_version(), "git_sha": sha,
            "source_sha256_16": h.hexdigest()[:16]}


def stream_ceiling(gib=4, reps=5):
    """Measured streaming-read ceiling: the best rate of a plain 16-byte read
    stream (libmla_probe.so) over a buffer of `gib` GiB, well beyond the
    256 MB Infinity Cache, over a few grid sizes."""
    import ctypes
    import numpy as np
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_22_amd", "libmla_probe.so"))
    L.mla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    L.mla_probe_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.random_(0, 255)
    stream = torch.cuda.current_stream()
    best, per = 0.0, {}
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks * 4, dtype=torch.int32, device="cuda")

        def run():
            assert L.mla_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream) == 0
        prewarm(lambda i: run(), 0.1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        per[blocks] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        best = max(best, per[blocks])
    del buf
    torch.cuda.empty_cache()
    return {"gbs": best, "by_grid": per, "bytes": nbytes,
            "kernel": "libmla_probe.so k_stream_read: 16-byte loads, 4 in flight per thread, 256 threads per group"}


def prewarm(fn, seconds=0.2):
    """Untimed calls fn(0), fn(1), ... for `seconds`: after an idle spell the
    clock ramps up over the first tens of milliseconds of sustained load, and
    calls measured there ran 10-20% slower."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def decode_call_leg(cfg, copies, n, ceiling=None):
    """The decode call alone (split + combine) at one workload: `copies` pool
    copies alternate so that the cache is not warm in the Infinity Cache;
    n calls, each timed with HIP events on the launch stream."""
    import numpy as np
    import torch
    from mla_latent_kv_22_amd import harness, inputs as I, mla
    print(f"[bench] building inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = I.make(cfg, 0)
    st = harness.DecodeStep(cfg, inp)
    st.step()
    pools = [st.pool] + [st.pool.clone() for _ in range(copies - 1)]
    stream = torch.cuda.current_stream()
    prewarm(lambda i: st.attend(pool=pools[i % copies]))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        st.attend(pool=pools[i % copies])
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    elem = 4 if cfg.dtype == "f32" else 2
    algo = int(np.sum(inp["seq_lens"].astype(np.int64))) * cfg.row_width * elem
    ms = float(np.mean(t))
    gbs = algo / (ms * 1e-3) / 1e9
    res = {"workload": f"{cfg.name}: B={cfg.batch} T={cfg.seq_len}{' (max, ragged U{%d..%d})' % (cfg.min_seq_len, cfg.seq_len) if cfg.min_seq_len else ''} "
                       f"H={cfg.num_heads} d_c={cfg.d_c} d_R={cfg.d_r} {cfg.dtype} page={cfg.page_size}",
           "fast_path": bool(mla.uses_fast_path(st.d, mla.OP_DECODE)),
           "algorithmic_bytes": algo, "decode_us": round(ms * 1e3, 2),
           "decode_us_p50_p95_p99": [round(float(np.percentile(t, p)) * 1e3, 2) for p in (50, 95, 99)],
           "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1), "calls": n, "cache_copies_rotated": copies}
    if ceiling:
        res["frac_of_measured_ceiling"] = round(gbs / ceiling, 4)
    del st, pools
    torch.cuda.empty_cache()
    return res


def projection_leg(n=64, calls=30):
    """Query compression (mla_project_q: W_DQ, W_UQ, then the absorption with
    W_UK) and output projection (mla_project_out: W_O) at the V3 shapes for
    one decode batch of n tokens.  Both stream their weights once per call;
    weight copies rotate so that they are not served from the 256 MB Infinity
    Cache."""
    import numpy as np
    import torch
    from mla_latent_kv_22_amd import harness, inputs as I, mla
    cfg = I.V3
    print("[bench] projection leg", file=sys.stderr, flush=True)
    inp = I.make(cfg, 0, with_rows=False)
    pj = I.projection_inputs(cfg, n, 3)
    d = harness.dims_for(cfg)
    dev = lambda x, dt="bf16": harness.to_device(x, dt)  # noqa: E731
    wq = [(dev(pj["w_dq"]), dev(pj["w_uq"]), dev(inp["w_uk"])) for _ in range(3)]
    wo = [dev(pj["w_o"]) for _ in range(2)]
    h, pos, o = dev(pj["h"]), dev(pj["positions"], "i32"), dev(pj["o"])
    q_abs = torch.empty((n, cfg.num_heads, cfg.row_width), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((n, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    wsq = torch.empty(mla.project_q_workspace_size(d, pj["d_cq"], n), dtype=torch.uint8, device="cuda")
    wso_n = mla.project_out_workspace_size(d, n)
    wso = torch.empty(max(wso_n, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        prewarm(fn)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])

    tq = timed(lambda i: mla.project_q(d, h, *wq[i % 3][:2], wq[i % 3][2], pos, q_abs, wsq))
    to = timed(lambda i: mla.project_out(d, o, wo[i % 2], y, wso if wso_n else None))
    bq = 2 * (pj["w_dq"].size + pj["w_uq"].size + inp["w_uk"].size)
    bo = 2 * pj["w_o"].size

    def leg(t, b, what):
        us = float(np.mean(t))
        return {"what": what, "weight_bytes": int(b), "us": round(us, 2),
                "us_p50_p95_p99": [round(float(np.percentile(t, p)), 2) for p in (50, 95, 99)],
                "weight_gbs": round(b / (us * 1e-6) / 1e9, 1), "frac_of_hbm_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del wq, wo
    torch.cuda.empty_cache()
    return {"workload": f"V3 shapes, {n} tokens: D={cfg.hidden}, d_cq={pj['d_cq']}, H={cfg.num_heads}, "
                        f"d_n+d_R={cfg.qk_head}, d_v={cfg.v_head}, bf16",
            "project_q": leg(tq, bq, "c_Q = W_DQ h, q = W_UQ c_Q, absorbed with W_UK"),
            "project_out": leg(to, bo, "y = W_O [o_1 | ... | o_H]")}


def calibrate():
    """A plain device copy of known size (1 GiB read + 1 GiB written, 3
    times): the FETCH_SIZE and WRITE_SIZE counters of this run give the
    factors from reported KiB to bytes."""
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {nbytes} bytes x 3", flush=True)


def _traffic(n_steps_note=""):
    """HBM bytes per decode call from committed rocprofv3 counter runs, or None
    when the counters are absent or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != _src_hash(DECODE_SRC):
        return None
    return t.get("bytes_per_decode_call")


def cpu_baseline(cfg, inp, budget_s=20.0):
    """Time the float64 oracle on a bounded sample of the same workload: whole
    sequences over all heads (the oracle's cost is linear in both), as many as
    fit in about budget_s seconds after timing the first one.  `cores` is the
    BLAS thread count the oracle ran with (the machine's CPU share sets it);
    `affinity_cpus` is what the scheduler would allow."""
    import numpy as np
    from tests._util import oracle_decode
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    t0 = time.perf_counter()
    oracle_decode(cfg, inp, [0])
    first = time.perf_counter() - t0
    n = int(max(1, min(cfg.batch, budget_s // max(first, 1e-3))))
    if n > 1:
        oracle_decode(cfg, inp, list(range(1, n)))
    dt = time.perf_counter() - t0
    sample_tokens = float(np.sum(inp["seq_lens"][:n].astype(np.int64)))
    return {"value": round(sample_tokens * cfg.row_width * 2 / dt / 1e9, 6), "unit": "GB/s", "cores": int(cores),
            "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"sequences 0..{n - 1} of {cfg.batch} ({int(sample_tokens)} cached tokens) x all {cfg.num_heads} "
                      f"heads, float64 NumPy, non-absorbed (per-head K and V materialised); rate = sample latent "
                      f"bytes / oracle seconds"}


def prefill_flops(cfg, lens):
    """Useful flops of the non-absorbed causal prefill: 2 (d_n + d_R + d_v) per
    (query, visible key, head), plus the K_C / V up-projection 2 d_c (d_n + d_v)
    per (token, head)."""
    pairs = sum(int(L) * (int(L) + 1) // 2 for L in lens)
    toks = sum(int(L) for L in lens)
    attn = 2.0 * (cfg.qk_nope + cfg.d_r + cfg.v_head) * cfg.num_heads * pairs
    proj = 2.0 * cfg.d_c * (cfg.qk_nope + cfg.v_head) * cfg.num_heads * toks
    return attn, proj


def prefill_leg(steps=5, warmup=10):
    """Cache write of every token + causal prefill at the v3_prefill workload.
    Each timed block follows 0.2 s and then `warmup` untimed calls of the same
    operation, so that the clocks have settled under the sustained load (the
    first calls after idle run up to 20% slower)."""
    import numpy as np
    import torch
    from mla_latent_kv_22_amd import harness, inputs as I
    cfg = I.PREFILL
    print(f"[bench] building inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = I.make(cfg, 0)
    pf = harness.Prefill(cfg, inp)
    stream = torch.cuda.current_stream()
    pf.write()
    pf.attend()
    torch.cuda.synchronize()

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    def settle(fn):
        prewarm(lambda i: fn())
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()

    settle(pf.write)
    w_ms = timed(pf.write)
    settle(pf.attend)
    a_ms = timed(pf.attend)
    attn, proj = prefill_flops(cfg, inp["seq_lens"])
    tf = (attn + proj) / (a_ms * 1e-3) / 1e12
    wflops = 2.0 * cfg.row_width * cfg.hidden * float(np.sum(inp["seq_lens"]))

    # chunked prefill: the second half of every sequence onto its cached first
    # half (mla_prefill_kv); useful work counts the new queries' visible keys
    # and the up-projection of every key
    from mla_latent_kv_22_amd import mla
    lens = inp["seq_lens"].astype(np.int64)
    pre = lens // 2
    new = lens - pre
    cu = inp["cu_seqlens"].astype(np.int64)
    idx = np.concatenate([np.arange(cu[b] + pre[b], cu[b + 1]) for b in range(len(lens))])
    q_new = pf.q[torch.as_tensor(idx, device=pf.q.device)].contiguous()
    cu_q = torch.as_tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32), device=pf.q.device)
    out_c = torch.empty((int(new.sum()),) + tuple(pf.out.shape[1:]), dtype=pf.out.dtype, device=pf.out.device)
    lse_c = torch.empty((int(new.sum()), cfg.num_heads), dtype=torch.float32, device=pf.out.device)
    ws_c = torch.empty(mla.prefill_workspace_size(pf.d, int(cu[-1])), dtype=torch.uint8, device=pf.q.device)

    def chunk():
        mla.prefill_kv(pf.d, q_new, pf.pool, pf.block_table, cu_q, pf.cu, int(cu[-1]), int(new.max()),
                       int(lens.max()), pf.w_uk, pf.w_uv, out_c, lse_c, ws_c)
    settle(chunk)
    c_ms = timed(chunk)
    c_pairs = float(sum(int(n) * int(p) + int(n) * (int(n) + 1) // 2 for n, p in zip(new, pre)))
    c_attn = 2.0 * (cfg.qk_nope + cfg.d_r + cfg.v_head) * cfg.num_heads * c_pairs
    c_proj = 2.0 * cfg.d_c * (cfg.qk_nope + cfg.v_head) * cfg.num_heads * float(lens.sum())
    c_tf = (c_attn + c_proj) / (c_ms * 1e-3) / 1e12
    return {"workload": f"{cfg.name}: {cfg.batch} x {cfg.seq_len} tokens, H={cfg.num_heads}, d_n=d_v={cfg.qk_nope}, "
                        f"d_R={cfg.d_r}, d_c={cfg.d_c}, D={cfg.hidden}, bf16, page={cfg.page_size}",
            "prefill_ms": round(a_ms, 4), "useful_tflop": round((attn + proj) / 1e12, 4),
            "tflops": round(tf, 1), "mfma_frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "write_cache_ms": round(w_ms, 4),
            "write_cache_tflops": round(wflops / (w_ms * 1e-3) / 1e12, 1),
            "chunked": {"workload": f"last {int(new[0])} tokens of each sequence onto its cached first {int(pre[0])}",
                        "ms": round(c_ms, 4), "useful_tflop": round((c_attn + c_proj) / 1e12, 4),
                        "tflops": round(c_tf, 1), "mfma_frac_of_bf16_peak": round(c_tf / BF16_PEAK_TFLOPS, 4)}}


def fp8_leg(steps=20):
    """The same decode step over the 8-bit cache (MLA_FLAG_FP8_CACHE): random
    E4M3 pages with power-of-two row scales, the step's B new rows quantized
    by the cache write.  Cache bytes per token: 576 codes + 4 scale bytes."""
    import numpy as np
    import torch
    from mla_latent_kv_22_amd import harness, inputs as I, mla
    cfg = I.V3
    inp = I.make(cfg, 0, with_rows=False)
    pages = I.fp8_pages(int(inp["num_pages"]), cfg.page_size, cfg.row_width, np.random.default_rng(0))
    st = harness.DecodeStep(cfg, inp, flags=mla.FLAG_FP8_CACHE, pool=torch.from_numpy(pages).to("cuda"))
    pools = [st.pool, st.pool.clone()]
    ws = torch.empty(mla.write_cache_workspace_size(st.d, cfg.batch), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def write(i):
        mla.write_cache(st.d, st.h, st.w_dkr, st.positions, st.slots, pools[i % 2], workspace=ws)

    def timed(fn, n):
        prewarm(fn, 0.1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    st.absorb()
    # alternating blocks of decode calls and of whole steps; medians of the blocks
    dec, stp = [], []
    for _ in range(3):
        dec.append(timed(lambda i: st.attend(pool=pools[i % 2]), steps))
        stp.append(timed(lambda i: (write(i), st.absorb(), st.attend(pool=pools[i % 2])), steps))
    dec_ms, step_ms = float(np.median(dec)), float(np.median(stp))
    tokens = int(np.sum(inp["seq_lens"].astype(np.int64)))
    cache_bytes = tokens * (cfg.row_width + 4)
    return {"workload": f"{cfg.name} over an 8-bit cache: B={cfg.batch} T={cfg.seq_len} H={cfg.num_heads}, "
                        f"E4M3 rows + float32 row scales, page={cfg.page_size}",
            "cache_bytes_per_call": cache_bytes,
            "decode_ms": round(dec_ms, 5), "decode_gbs": round(cache_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "decode_tokens_per_s": round(cfg.batch / (dec_ms * 1e-3), 1),
            "step_ms": round(step_ms, 5), "step_tokens_per_s": round(cfg.batch / (step_ms * 1e-3), 1),
            "launch": "eager, one stream"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit cache leg")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a HIP graph (one per cache copy) instead of launching it eagerly")
    ap.add_argument("--no-graph", action="store_true", help="eager launches (the default)")
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (the clock ramps up under load)")
    ap.add_argument("--no-legs", action="store_true", help="skip the other decode workloads and the read ceiling")
    ap.add_argument("--calibrate", action="store_true", help="only the counter-calibration copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); multi-GPU runs are not part of this "
              f"library's measurements", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mla_latent_kv_22_amd import harness, inputs as I, mla

    if args.calibrate:
        calibrate()
        return
    mla.lib()
    if args.workload == "v3_decode_fp8":
        # 8-bit cache leg only (profiling runs): one JSON line
        print(json.dumps({"metric": "MLA decode over an 8-bit latent cache", "n_gpus": 1, **fp8_leg(args.steps)}),
              flush=True)
        return
    cfg = I.CONFIGS[args.workload]
    if cfg.prefill:
        # prefill only (profiling runs): one JSON line for the prefill leg
        print(json.dumps({"metric": "MLA causal prefill useful TFLOP/s", "n_gpus": 1, **prefill_leg(args.steps, args.warmup)}),
              flush=True)
        return
    print(f"[bench] building inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = I.make(cfg, 0)
    st = harness.DecodeStep(cfg, inp)
    # two pool copies, alternated per step, so no step finds the cache warm in
    # the 256 MB Infinity Cache from the step before
    pools = [st.pool, st.pool.clone()]
    stream = torch.cuda.current_stream()
    algo_bytes = int(np.sum(inp["seq_lens"].astype(np.int64))) * cfg.row_width * 2

    # one stream: mla_write_absorb (the cache write and the absorption in one
    # launch), then the decode.  A side stream for a separate cache write
    # (concurrent with the absorption) measured 17 us slower per step in a
    # graph, the cost of joining the two streams before the decode.  Eager
    # launches by default: the host stays ahead of the GPU, so the kernels of
    # consecutive steps run back to back, while graph replays left about 8 us
    # idle between one replay and the next (kernel trace).
    def step(i):
        st.step(pool=pools[i % 2])

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    if args.graph and not args.no_graph:
        # one HIP graph per cache copy: the step's three launches replay without
        # host launch gaps (the kernels allocate nothing and take no host sync)
        graphs = []
        for k in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st.step(pool=pools[k])
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):  # noqa: F811
            graphs[i % 2].replay()
    # the timed step runs untimed for --prewarm-s seconds (the clock ramps up
    # under load), then W warmup steps
    prewarm(step, args.prewarm_s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] warm", file=sys.stderr, flush=True)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-phase timing: each phase alone, same stream, per-call events
    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record(stream)
            fn(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    # the decode first, while the clock is where the step loop left it; the
    # short projection calls after it
    t_decode = timed(lambda i: st.attend(pool=pools[i % 2]), args.steps)
    t_write = timed(lambda i: st.write(pool=pools[i % 2]), args.steps)
    t_absorb = timed(lambda i: st.absorb(), args.steps)
    t_wa = timed(lambda i: st.write_absorb(pool=pools[i % 2]), args.steps)
    dec_ms = float(np.mean(t_decode))

    flops = 2.0 * cfg.num_heads * (cfg.row_width + cfg.d_c) * float(np.sum(inp["seq_lens"]))
    achieved = algo_bytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": "MLA decode latent-cache GB/s (% HBM peak) + tokens/s at B=64,T=8k,H=128",
        "value": round(algo_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent rows and hidden states, N(0,0.02^2) weights)",
        "config": {"workload": f"{cfg.name}: B={cfg.batch} T={cfg.seq_len}{' (max, ragged)' if cfg.min_seq_len else ''} "
                               f"H={cfg.num_heads} d_c={cfg.d_c} d_R={cfg.d_r} d_v={cfg.v_head} bf16 page={cfg.page_size}",
                   "batch": cfg.batch, "context": cfg.seq_len, "heads": cfg.num_heads,
                   "step": "write_absorb (cache write of B rows + absorb_q, one launch), decode(split + combine), "
                           "one stream",
                   "launch": "hip graph per step" if args.graph and not args.no_graph else "eager, one stream",
                   "cache_copies_rotated": 2},
        "pct_hbm_peak": round(100.0 * algo_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.batch / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": algo_bytes,
        "phases_ms": {"write_absorb": round(float(np.mean(t_wa)), 5),
                      "write_cache": round(float(np.mean(t_write)), 5), "absorb_q": round(float(np.mean(t_absorb)), 5),
                      "decode": round(dec_ms, 5),
                      "decode_p50_p95_p99": [round(float(np.percentile(t_decode, p)), 5) for p in (50, 95, 99)]},
        "roofline": {"kernel": "mla_decode (split-T pass + combine, one stream)", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(),
                     "mfma_tflops": round(flops / (dec_ms * 1e-3) / 1e12, 1),
                     "mfma_frac_of_bf16_peak": round(flops / (dec_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_legs:
        print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
        ceil = stream_ceiling()
        res["measured_read_ceiling"] = ceil
        res["roofline"]["measured_ceiling_gbs"] = ceil["gbs"]
        res["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["gbs"], 4)
        res["decode_workloads"] = [decode_call_leg(I.TINY, 1, 50, ceil["gbs"]),
                                   decode_call_leg(I.V2LITE, 8, 100, ceil["gbs"]),
                                   decode_call_leg(I.RAGGED, 1, 50, ceil["gbs"])]
        res["projections"] = projection_leg()
    res["conditions"] = conditions()
    if not args.no_prefill:
        res["prefill"] = prefill_leg()
    if not args.no_fp8:
        res["fp8_cache"] = fp8_leg()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
