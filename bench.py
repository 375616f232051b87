"""Benchmark of the int8-KV attention hot path on one MI355X.

One step = one verify call (attn_verify_q8 + attn_reduce_partials) on the
verify-window workload (24 Q / 4 KV heads, head_dim 256, context 20,676, 8
sequential rows) followed by one prompt call (attn_prompt_q8) on the prompt
chunk (12 Q / 1 KV head, head_dim 256, 32,768-token int8 context, 2,048 causal
queries).  Inputs are seeded synthetic data resident in HBM before timing, in
several rotating copies so that the 256 MB Infinity Cache cannot serve
repeats.  Durations come from HIP events recorded on the library's stream:
around each whole verify call (attention kernel + reducer, nothing recorded
between them) and each prompt call, and on alternate steps one more event after
the attention kernel, which times it alone for its roofline.  The GPU is held by
a spin kernel while the timed launches are queued so that host submission
latency does not enter them.  The practical HBM read ceiling (a plain 1 GiB
read by the library's attnq8_stream_read) is reported beside the 8 TB/s peak.

Prints one JSON line.  Other modes:
  --copy-calibration   run only plain device copies of a known size (for
                       scaling the FETCH_SIZE / WRITE_SIZE counters)
  --sweep              the shared-scan comparison over context lengths: the
                       verify call (8 rows) with one row per workgroup (every
                       row scans K/V on its own) against row groups of 4 and 8
                       rows, at 24 Q / 4 KV heads, head_dim 256, contexts
                       2,048 / 4,096 / 20,676 / 32,768 and head_dim 128 at
                       8,192; one JSON line per cell
  --oracle-times       the fp64 oracle per workload on the host (bounded
                       samples, no GPU) and the tests' pure-Python brute force
                       on the tiny verify; one JSON line per workload
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "verify-attn KV GB/s (% HBM peak); prompt-attn TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--verify-workload", default="verify_window")
    ap.add_argument("--prompt-workload", default="prompt_chunk")
    ap.add_argument("--no-prompt", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows-per-group", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--oracle-times", action="store_true",
                    help="time the fp64 oracle per workload on the host (no GPU)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counter results are valid only for the sources they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_int8_quantized_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """Counter-derived HBM bytes per launch, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("kernels", {}).get(kernel_key)


def copy_calibration():
    import torch

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "bytes_per_copy": COPY_BYTES, "copies": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        sweep(args)
        return
    if args.oracle_times:
        oracle_times()
        return

    import torch

    import workloads as W
    from attention_int8_quantized_amd import ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wv = W.WORKLOADS[args.verify_workload]
    wp = W.WORKLOADS[args.prompt_workload]

    # ---------------- inputs (host -> device, then device-side copies) ----------
    log(f"generating {wv.name}")
    iv = W.generate(wv)
    v_host = [iv.q, iv.k_codes, iv.k_scales, iv.v_codes, iv.v_scales]
    kv_bytes_v = sum(x.nbytes for x in v_host[1:])
    nv = max(1, min(64, int(args.rotate_bytes // max(kv_bytes_v, 1)) + 1))
    base = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in v_host]
    vbufs = [base] + [[t.clone() for t in base] for _ in range(nv - 1)]
    S = args.splits or ops.verify_splits(wv.n_q_heads, wv.n_kv_heads, wv.head_dim, wv.ctx_len,
                                         wv.n_rows, args.rows_per_group)
    ws = torch.empty(ops.workspace_bytes(wv.n_rows, wv.n_q_heads, wv.head_dim, S), dtype=torch.uint8,
                     device=dev)
    vout = torch.empty((wv.n_rows, wv.n_q_heads, wv.head_dim), dtype=torch.float32, device=dev)

    pbufs = []
    if not args.no_prompt:
        log(f"generating {wp.name}")
        ip = W.generate(wp)
        p_host = [ip.q, ip.k_codes, ip.k_scales, ip.v_codes, ip.v_scales]
        pbytes = sum(x.nbytes for x in p_host)
        npb = max(1, min(16, int(0.35e9 // pbytes) + 1))
        pbase = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in p_host]
        pbufs = [pbase] + [[t.clone() for t in pbase] for _ in range(npb - 1)]
        pout = torch.empty((wp.n_queries, wp.n_q_heads, wp.head_dim), dtype=torch.float32,
                           device=dev)
    torch.cuda.synchronize()

    def verify_call(i):
        q, kc, ks, vc, vs = vbufs[i % len(vbufs)]
        ops.verify_partials(q, kc, ks, vc, vs, ctx_len=wv.ctx_len,
                            rows_per_group=args.rows_per_group, n_splits=S, workspace=ws)

    def reduce_call():
        ops.reduce_partials(ws, wv.n_rows, wv.n_q_heads, wv.head_dim, S, out=vout)

    def prompt_call(i):
        q, kc, ks, vc, vs = pbufs[i % len(pbufs)]
        ops.prompt(q, kc, ks, vc, vs, q_pos0=wp.pos0, kv_len=wp.kv_len, out=pout)

    # ---------------- warmup -----------------------------------------------------
    for i in range(args.warmup):
        verify_call(i)
        reduce_call()
        if pbufs:
            prompt_call(i)
    torch.cuda.synchronize()
    verify_call(0)
    verify_path = ops.last_path()
    prompt_path = None
    if pbufs:
        prompt_call(0)
        prompt_path = ops.last_path()
    torch.cuda.synchronize()

    # ---------------- timed region ------------------------------------------------
    K = args.steps
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [[E() for _ in range(4)] for _ in range(K)]
    t_start, t_end = E(), E()
    torch.cuda.synchronize()
    # hold the GPU while the launches are queued (~50 us of host time per step)
    torch.cuda._sleep(int(2.4e9 * (0.06e-3 * K + 0.02)))
    wall0 = time.perf_counter()
    t_start.record()
    # Events bracket the verify call (kernel + reducer) and the prompt call of
    # every step; on odd steps one more event between the attention kernel and
    # the reducer times the kernel alone (its roofline).  The call's time is
    # taken from the even steps, which have nothing recorded inside the call.
    for i in range(K):
        e = ev[i]
        e[0].record()
        verify_call(i + 1)
        if i % 2 == 1 or K < 2:
            e[1].record()
        reduce_call()
        e[2].record()
        if pbufs:
            prompt_call(i + 1)
        e[3].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    odd = [i for i in range(K) if i % 2 == 1 or K < 2]
    even = [i for i in range(K) if i % 2 == 0]
    k1 = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in odd]) * 1e-3  # s
    kv = np.array([ev[i][0].elapsed_time(ev[i][2]) for i in even]) * 1e-3
    kp = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]) * 1e-3
    step_ms = t_start.elapsed_time(t_end) / K

    # KV bytes of the grouping the library used (rows_per_group 0 = its choice)
    m = re.search(r"rows_per_group(\d+)", verify_path or "")
    rg_used = int(m.group(1)) if m else (args.rows_per_group or wv.rows_per_group)
    vbytes = wv.visible_kv_bytes(rg_used)
    verify_s = float(np.mean(kv))
    gbs = vbytes / verify_s / 1e9
    k1_mean = float(np.mean(k1))
    k1_gbs = vbytes / k1_mean / 1e9
    tr_v = load_traffic("verify")

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-kv/fp16-mfma/fp32",
        "data": "synthetic (seeded N(0,1), int8 block-32 quantised KV)",
        "config": {
            "workload": wv.name,
            "verify": {**W.describe(wv), "rows_per_group": rg_used, "splits": S,
                       "rotating_copies": len(vbufs), "path": verify_path},
            "parallelism": "single-gpu",
        },
        "verify": {
            "us_per_call": round(verify_s * 1e6, 3),
            "kernel_us": round(k1_mean * 1e6, 3),
            "reduce_us": round((verify_s - k1_mean) * 1e6, 3),
            "kv_bytes": vbytes,
            "unique_kv_bytes": wv.unique_kv_bytes(),
            "gbs": round(gbs, 2),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "kernel": "attend_q8_kernel (verify)",
            "bound": "hbm",
            "achieved": round(k1_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
            "traffic": tr_v,
        },
    }
    if pbufs:
        flops = wp.algorithmic_flops()
        kp_mean = float(np.mean(kp))
        tf = flops / kp_mean / 1e12
        res["prompt"] = {
            "workload": wp.name,
            "config": W.describe(wp),
            "path": prompt_path,
            "ms_per_call": round(kp_mean * 1e3, 4),
            "tflops": round(tf, 2),
            "frac_mfma": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "rotating_copies": len(pbufs),
        }
        res["prompt_roofline"] = {
            "kernel": "attend_own_q8_kernel (prompt)",
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prompt"),
        }
    res["host_wall_s"] = round(wall, 3)
    ceil = read_ceiling(ops, dev)
    res["read_ceiling"] = ceil
    res["verify"]["frac_of_read_ceiling"] = round(gbs / ceil["gbs"], 4)
    res["verify"]["kernel_frac_of_read_ceiling"] = round(k1_gbs / ceil["gbs"], 4)
    if not args.no_append:
        res["kv_append"] = time_append(ops, dev, min(K, 20), args.warmup)
        res["verify_head"] = time_head(ops, dev, min(K, 20), args.warmup)
        res.update(time_f16kv(ops, dev, wv, wp, min(K, 20), args.warmup, not args.no_prompt))

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wv, iv)

    print(json.dumps(res), flush=True)


def read_ceiling(ops, dev, nbytes=1 << 30, reps=10):
    """The practical HBM read rate: the library's plain read kernel over 1 GiB
    (16-byte loads, every byte read once), median of `reps` launches."""
    import torch

    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(ops.STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    for _ in range(3):
        ops.stream_read(buf, sink)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(reps)]
    for a, b in ev:
        a.record()
        ops.stream_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    gbs = nbytes / t / 1e9
    del buf
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "1 GiB read once with 16-byte loads (attnq8_stream_read), median of 10"}


def _host_threads():
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        return max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        return os.cpu_count()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_times():
    """The fp64 oracle per workload on the host, each on a bounded sample timed
    for a few seconds, and the pure-Python brute force of the tests on the tiny
    verify; one JSON line per workload."""
    import oracle
    import workloads as W

    host = {"cpu": _cpu_model(), "cpu_count": os.cpu_count(), "blas_threads": _host_threads()}
    for name, w in W.WORKLOADS.items():
        inp = W.generate(w)
        if w.kind == "verify":
            # one KV head with its query heads, all rows
            q = inp.q[:, : w.group]
            call = lambda: oracle.verify(q, inp.k_codes[:1], inp.k_scales[:1],  # noqa: E731
                                         inp.v_codes[:1], inp.v_scales[:1], w.ctx_len)
            frac = 1.0 / w.n_kv_heads
        else:
            rows = list(range(0, w.n_queries, max(1, w.n_queries // 16)))
            call = lambda: oracle.prompt(inp.q, inp.k_codes, inp.k_scales,  # noqa: E731
                                         inp.v_codes, inp.v_scales, w.pos0, rows=rows)
            frac = len(rows) / w.n_queries
        reps, t0 = 0, time.perf_counter()
        while reps < 1 or (time.perf_counter() - t0 < 3.0 and reps < 1000):
            call()
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        full_s = dt / frac
        line = {"mode": "oracle-times", "workload": name, "sample_s": round(dt, 4),
                "sample_fraction": round(frac, 5), "whole_workload_s": round(full_s, 5),
                "algorithmic_gflops": round(w.algorithmic_flops() * frac / dt / 1e9, 3), **host}
        print(json.dumps(line), flush=True)
    # the pure-Python brute force of the tests on the tiny verify, one core
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import bruteforce

    w = W.TINY_VERIFY
    inp = W.generate(w)
    pos = [w.ctx_len + r for r in range(w.n_rows)]
    t0 = time.perf_counter()
    bruteforce.attention(inp.q.tolist(), pos, inp.k_codes.tolist(), inp.k_scales.tolist(),
                         inp.v_codes.tolist(), inp.v_scales.tolist())
    print(json.dumps({"mode": "oracle-times", "workload": w.name, "brute_force_s":
                      round(time.perf_counter() - t0, 3), "cores": 1, **host}), flush=True)


def cpu_baseline(wv, iv):
    """The fp64 oracle on the host, on a bounded sample of the verify workload."""
    import oracle

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = os.cpu_count()
    # sample: all query vectors of the first KV head (a quarter of the work)
    heads = list(range(wv.group))
    q = iv.q[:, heads]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify(q, iv.k_codes[:1], iv.k_scales[:1], iv.v_codes[:1], iv.v_scales[:1],
                      wv.ctx_len)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 5000:
            break
    dt = (time.perf_counter() - t0) / reps
    sample_bytes = wv.visible_kv_bytes() / wv.n_kv_heads
    return {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{wv.name}: KV head 0 with its {wv.group} Q heads x {wv.n_rows} rows "
                  f"({sample_bytes} KV bytes), {reps} repetitions of {dt:.3f} s",
    }


# KV append measured beside the attention: the K and V rows of a 32,768-token
# context, 4 KV heads, head_dim 256, fp32 rows in, int8 blocks + fp16 scales out.
APPEND_SHAPE = (32768, 4, 256)


def time_append(ops, dev, steps, warmup):
    import torch

    T, H, hd = APPEND_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rows = [[torch.randn((T, H, hd), generator=g, device=dev) for _ in range(2)] for _ in range(2)]
    kc = torch.empty((H, T, hd), dtype=torch.int8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((H, T, hd // 32), dtype=torch.float16, device=dev)
    vs = torch.empty_like(ks)

    def call(i):
        k, v = rows[i % 2]
        ops.kv_append(k, kc, ks, 0, v, vc, vs)

    for i in range(warmup):
        call(i)
    call(0)
    path = ops.last_path()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(steps)]
    torch.cuda._sleep(int(2.4e9 * (0.05e-3 * steps + 0.02)))
    for i in range(steps):
        ev[i][0].record()
        call(i + 1)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    n = T * H * hd
    moved = 2 * (n * 4 + n + (n // 32) * 2)  # K and V: fp32 rows read, codes + scales written
    gbs = moved / t / 1e9
    return {
        "workload": f"K and V rows of {T} tokens x {H} KV heads x head_dim {hd}, fp32",
        "path": path,
        "us_per_call": round(t * 1e6, 3),
        "bytes": moved,
        "gbs": round(gbs, 1),
        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "steps": steps,
        "traffic": load_traffic("append"),
    }


def _events_mean(call, steps, warmup):
    import torch

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(steps)]
    torch.cuda._sleep(int(2.4e9 * (0.05e-3 * steps + 0.02)))
    for i in range(steps):
        ev[i][0].record()
        call(i + 1)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3


def time_f16kv(ops, dev, wv, wp, steps, warmup, with_prompt):
    """The verify and prompt workloads over an fp16 K/V cache (the same seeded
    draws rounded to fp16 instead of quantised), measured beside the int8 path."""
    import torch

    import workloads as W

    out = {}
    iv = W.generate_f16kv(wv)
    base = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (iv.q, iv.k, iv.v)]
    kvb = base[1].numel() * 2 + base[2].numel() * 2
    copies = [base] + [[t.clone() for t in base] for _ in range(max(0, int(1.1e9 // kvb)))]
    S = ops.verify_splits(wv.n_q_heads, wv.n_kv_heads, wv.head_dim, wv.ctx_len, wv.n_rows, 0)
    ws = torch.empty(ops.workspace_bytes(wv.n_rows, wv.n_q_heads, wv.head_dim, S),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((wv.n_rows, wv.n_q_heads, wv.head_dim), dtype=torch.float32, device=dev)

    def vcall(i):
        q, k, v = copies[i % len(copies)]
        ops.verify_f16kv_partials(q, k, v, ctx_len=wv.ctx_len, n_splits=S, workspace=ws)

    vcall(0)
    vpath = ops.last_path()
    t = _events_mean(vcall, steps, warmup)
    # fp16 K and V bytes of the grouping the library chose
    m = re.search(r"rows_per_group(\d+)", vpath or "")
    rg = int(m.group(1)) if m else wv.rows_per_group
    vis = wv.visible_kv_bytes(rg) // (2 * (wv.head_dim + wv.head_dim // 16)) * 4 * wv.head_dim
    out["verify_f16kv"] = {
        "workload": f"{wv.name} over an fp16 cache",
        "path": vpath,
        "kernel_us": round(t * 1e6, 3),
        "kv_bytes": vis,
        "gbs": round(vis / t / 1e9, 1),
        "frac_hbm": round(vis / t / 1e9 / HBM_PEAK_GBS, 4),
        "rotating_copies": len(copies),
        "traffic": load_traffic("verify_f16kv"),
    }
    ops.reduce_partials(ws, wv.n_rows, wv.n_q_heads, wv.head_dim, S, out=o)
    del copies, base
    if with_prompt:
        ip = W.generate_f16kv(wp)
        pb = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (ip.q, ip.k, ip.v)]
        pout = torch.empty((wp.n_queries, wp.n_q_heads, wp.head_dim), dtype=torch.float32,
                           device=dev)
        pcopies = [pb] + [[t.clone() for t in pb] for _ in range(7)]

        def pcall(i):
            q, k, v = pcopies[i % len(pcopies)]
            ops.prompt_f16kv(q, k, v, q_pos0=wp.pos0, kv_len=wp.kv_len, out=pout)

        pcall(0)
        ppath = ops.last_path()
        tp = _events_mean(pcall, max(3, steps // 4), 1)
        tf = wp.algorithmic_flops() / tp / 1e12
        out["prompt_f16kv"] = {
            "workload": f"{wp.name} over an fp16 cache",
            "path": ppath,
            "ms_per_call": round(tp * 1e3, 4),
            "tflops": round(tf, 2),
            "frac_mfma": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prompt_f16kv"),
        }
    return out


# The verify head measured beside the attention: greedy token and top
# probability of 5 rows of 248,320 fp32 logits (the sampler page's benchmark
# shape), several rotating copies so that the rows come from HBM.
HEAD_SHAPE = (5, 248320)


def time_head(ops, dev, steps, warmup):
    import torch

    rows, V = HEAD_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    copies = [torch.randn((rows, V), generator=g, device=dev) * 3 for _ in range(64)]
    ws = torch.zeros(ops.head_workspace_bytes(rows, V), dtype=torch.uint8, device=dev)
    tok = torch.empty(rows, dtype=torch.int32, device=dev)
    top = torch.empty(rows, dtype=torch.float32, device=dev)

    def call(i):
        ops.verify_head_greedy(copies[i % len(copies)], workspace=ws, token=tok, top_prob=top)

    for i in range(warmup):
        call(i)
    call(0)
    path = ops.last_path()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(steps)]
    torch.cuda._sleep(int(2.4e9 * (0.05e-3 * steps + 0.02)))
    for i in range(steps):
        ev[i][0].record()
        call(i + 1)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    moved = rows * V * 4
    return {
        "workload": f"{rows} rows x {V} fp32 logits: greedy token + top probability",
        "path": path,
        "us_per_call": round(t * 1e6, 3),
        "bytes": moved,
        "gbs": round(moved / t / 1e9, 1),
        "frac_hbm": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
        "steps": steps,
        "traffic": load_traffic("head"),
    }


# The context sweep of "perf(gfx1100): share Q8 KV scans across verifier rows",
# Kernel evidence: (n_q_heads, n_kv_heads, head_dim, ctx).  The page gives the
# head_dim 128 screen without its head counts; it is taken at the same 24 / 4.
SWEEP_SHAPES = [(24, 4, 256, 2048), (24, 4, 256, 4096), (24, 4, 256, 20676),
                (24, 4, 256, 32768), (24, 4, 128, 8192)]
SWEEP_ROWS = 8
SWEEP_GROUPS = (1, 4, 8)


def time_verify(ops, bufs, w, rows_per_group, steps, warmup):
    """Mean durations (s) over rotating inputs: the attention kernel alone, and the
    rest of the verify call (reducer and the launch gap before it)."""
    import torch

    S = ops.verify_splits(w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_len, w.n_rows,
                          rows_per_group)
    ws = torch.empty(ops.workspace_bytes(w.n_rows, w.n_q_heads, w.head_dim, S),
                     dtype=torch.uint8, device=bufs[0][0].device)
    out = torch.empty((w.n_rows, w.n_q_heads, w.head_dim), dtype=torch.float32,
                      device=ws.device)

    def call(i):
        q, kc, ks, vc, vs = bufs[i % len(bufs)]
        ops.verify_partials(q, kc, ks, vc, vs, ctx_len=w.ctx_len,
                            rows_per_group=rows_per_group, n_splits=S, workspace=ws)

    def reduce():
        ops.reduce_partials(ws, w.n_rows, w.n_q_heads, w.head_dim, S, out=out)

    for i in range(warmup):
        call(i)
        reduce()
    call(0)
    path = ops.last_path()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [[E() for _ in range(3)] for _ in range(steps)]
    torch.cuda._sleep(int(2.4e9 * (0.05e-3 * steps + 0.02)))
    # (as in the main run: the kernel alone on odd steps, the whole call on even ones)
    for i in range(steps):
        ev[i][0].record()
        call(i + 1)
        if i % 2 == 1 or steps < 2:
            ev[i][1].record()
        reduce()
        ev[i][2].record()
    torch.cuda.synchronize()
    odd = [e for i, e in enumerate(ev) if i % 2 == 1 or steps < 2]
    even = [e for i, e in enumerate(ev) if i % 2 == 0]
    k1 = float(np.mean([e[0].elapsed_time(e[1]) for e in odd])) * 1e-3
    k2 = float(np.mean([e[0].elapsed_time(e[2]) for e in even])) * 1e-3 - k1
    return k1, k2, S, path


def sweep(args):
    import torch

    import workloads as W
    from attention_int8_quantized_amd import ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = min(args.steps, 30)
    for hq, hkv, hd, ctx in SWEEP_SHAPES:
        w = W.VerifyWorkload(f"sweep_hd{hd}_ctx{ctx}", hq, hkv, hd, ctx, SWEEP_ROWS, SWEEP_ROWS)
        inp = W.generate(w)
        host = [inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales]
        kv_bytes = sum(x.nbytes for x in host[1:])
        n = max(1, min(256, int(args.rotate_bytes // kv_bytes) + 1))
        base = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in host]
        bufs = [base] + [[t.clone() for t in base] for _ in range(n - 1)]
        torch.cuda.synchronize()
        cells = {}
        for rg in SWEEP_GROUPS:
            k1, k2, S, path = time_verify(ops, bufs, w, rg, steps, args.warmup)
            cells[rg] = (k1, k2, S, path)
        t1 = cells[1][0] + cells[1][1]
        for rg in SWEEP_GROUPS:
            k1, k2, S, path = cells[rg]
            tot = k1 + k2
            line = {
                "mode": "sweep", "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": hd,
                "ctx": ctx, "rows": SWEEP_ROWS, "rows_per_group": rg, "splits": S,
                "path": path, "kernel_us": round(k1 * 1e6, 3), "reduce_us": round(k2 * 1e6, 3),
                "total_us": round(tot * 1e6, 3),
                "visible_kv_gbs": round(w.visible_kv_bytes(rg) / tot / 1e9, 1),
                "unique_kv_gbs": round(w.unique_kv_bytes() / tot / 1e9, 1),
                "speedup_vs_rows_per_group_1": round(t1 / tot, 3),
                "rotating_copies": n, "steps": steps,
            }
            print(json.dumps(line), flush=True)
        del bufs, base
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
