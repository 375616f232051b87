"""Benchmark of the int8-KV attention hot path on one MI355X.

One step = one verify call (attn_verify_q8 + attn_reduce_partials) on the
long-context verify workload (24 Q / 4 KV heads, head_dim 256, context 131,072,
4 sequential rows, 1% of K positions x8) followed by one prompt call
(attn_prompt_q8) on the prompt chunk (12 Q / 1 KV head, head_dim 256,
32,768-token int8 context, 2,048 causal queries).  The headline `value` is the
verify call's KV GB/s; the prompt's TFLOP/s is reported beside it.  The other
verify configurations (the verify window, the verify batch with the pages' R4
row groups, with the library's own grouping and as one group of all 32 rows,
the tiny verify) are timed in
the same run and reported in `verify_configs`.

Inputs are seeded synthetic data resident in HBM before timing, each workload
in rotating copies of at least 1 GB (four times the 256 MB Infinity Cache)
so that repeats come from HBM.  Durations come from HIP events recorded on the
library's stream: around each whole verify call (attention kernel + reducer,
nothing recorded between them) and each prompt call, and on alternate steps one
more event after the attention kernel, which times it and the reducer after it
(with that launch's dispatch gap) separately.  An event
between two launches adds several microseconds of its own, so the attention
kernel and the reducer are also timed each alone, launched back to back after
the steps (events around the region divided by its launches: the GPU time per
launch with its dispatch gap and no per-launch event latency); the verify
roofline's launch duration is the attention kernel's.
The GPU is kept busy by plain read kernels while the timed launches are queued so that
host submission latency does not enter them.  The practical HBM read ceiling
(a plain 1 GiB read by the library's attnq8_stream_read) is reported beside the
8 TB/s peak.

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
  --summarize-trace F  per-kernel durations from a rocprofv3 kernel-trace CSV,
                       grouped by kernel and grid, the first --skip-first
                       launches of each group (the warm-up) left out; a
                       markdown table (no GPU)
  --summarize-pmc F..  per-dispatch means of the counters in rocprofv3 --pmc
                       counter-collection CSVs, by kernel and grid; a markdown
                       table (no GPU)
  --traffic-from DIR   HBM bytes per launch from the FETCH_SIZE and WRITE_SIZE
                       passes over bench.py and over --copy-calibration (CSVs
                       under DIR/FETCH_SIZE, DIR/WRITE_SIZE, DIR/FETCH_SIZE_copy,
                       DIR/WRITE_SIZE_copy), scaled by the copy's known size;
                       prints a markdown table and, with --write-traffic,
                       writes profiles/traffic.json for these sources (no GPU)
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
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--verify-workload", default="long_verify")
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
    ap.add_argument("--no-extra-verify", action="store_true",
                    help="skip the other verify configurations")
    ap.add_argument("--summarize-trace", default=None,
                    help="a rocprofv3 *_kernel_trace.csv to summarise (no GPU)")
    ap.add_argument("--summarize-pmc", nargs="+", default=None)
    ap.add_argument("--traffic-from", default=None)
    ap.add_argument("--write-traffic", action="store_true")
    ap.add_argument("--tail", type=int, default=0,
                    help="--summarize-trace: only the last N launches of each group")
    ap.add_argument("--skip-first", type=int, default=6,
                    help="launches per (kernel, grid) group left out by --summarize-trace")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def strip_comments(src: str) -> str:
    """C++ source text without its comments, whitespace runs collapsed to one
    space (string and character literals kept as they are)."""
    out = []
    i, n = 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the HIP sources' code (comments and layout left out): counter
    results are valid only for the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_int8_quantized_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
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
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.traffic_from:
        traffic_from(args.traffic_from, args.write_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.skip_first, args.tail)
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
    vbufs = rotating_copies([iv.q, iv.k_codes, iv.k_scales, iv.v_codes, iv.v_scales], dev,
                            args.rotate_bytes)
    S = args.splits or ops.verify_splits(wv.n_q_heads, wv.n_kv_heads, wv.head_dim, wv.ctx_len,
                                         wv.n_rows, args.rows_per_group)
    ws = torch.empty(ops.workspace_bytes(wv.n_rows, wv.n_q_heads, wv.head_dim, S), dtype=torch.uint8,
                     device=dev)
    vout = torch.empty((wv.n_rows, wv.n_q_heads, wv.head_dim), dtype=torch.float32, device=dev)

    pbufs = []
    if not args.no_prompt:
        log(f"generating {wp.name}")
        ip = W.generate(wp)
        pbufs = rotating_copies([ip.q, ip.k_codes, ip.k_scales, ip.v_codes, ip.v_scales], dev,
                                args.rotate_bytes)
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

    verify_call(0)
    verify_path = ops.last_path()
    prompt_path = None
    if pbufs:
        prompt_call(0)
        prompt_path = ops.last_path()
    hold = Hold(ops, dev)

    # ---------------- warmup, then the timed region --------------------------------
    # The warm-up steps run back to back, so that the clocks have settled when
    # timing starts (after an idle gap the first launches run up to 25% slower);
    # a short busy hold keeps the GPU working while the first timed launches are
    # queued.
    K = args.steps
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [[E() for _ in range(4)] for _ in range(K)]
    t_start, t_end = E(), E()
    torch.cuda.synchronize()
    for i in range(args.warmup):
        verify_call(i)
        reduce_call()
        if pbufs:
            prompt_call(i)
    torch.cuda.synchronize()
    hold(1e-3)
    wall0 = time.perf_counter()
    t_start.record()
    # Events bracket the verify call (kernel + reducer) and the prompt call of
    # every step; on odd steps one more event between the attention kernel and
    # the reducer times the kernel and the reducer separately.  The call's time
    # is taken from the even steps, which have nothing recorded inside the call.
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

    # Back-to-back regions after the steps (events around each region, divided
    # by its launches; a kernel bracketed by its own events also carries the
    # event's latency): whole calls (attention kernel + reducer, no event
    # inside), the reducer alone, and last the attention kernel alone over the
    # rotating inputs, whose launch duration is the roofline's.
    KR = max(K, 10)
    r0, r1 = E(), E()

    def region(body):
        torch.cuda.synchronize()
        hold(60e-6 * KR + 1e-3)
        r0.record()
        for i in range(KR):
            body(i + 1)
        r1.record()
        torch.cuda.synchronize()
        return r0.elapsed_time(r1) / KR * 1e-3  # s

    cr_mean = region(lambda i: (verify_call(i), reduce_call()))
    rr_mean = region(lambda i: reduce_call())  # (the partials of the last call)
    kr_mean = region(verify_call)

    odd = [i for i in range(K) if i % 2 == 1 or K < 2]
    even = [i for i in range(K) if i % 2 == 0]
    k1 = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in odd]) * 1e-3  # s
    kr = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in odd]) * 1e-3  # the reducer after it
    kv = np.array([ev[i][0].elapsed_time(ev[i][2]) for i in even]) * 1e-3
    kp = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]) * 1e-3
    step_ms = t_start.elapsed_time(t_end) / K

    # KV bytes of the grouping the library used (rows_per_group 0 = its choice)
    rg_used = rows_per_group_of(verify_path, args.rows_per_group or wv.rows_per_group)
    vbytes = wv.visible_kv_bytes(rg_used)
    verify_s = float(np.mean(kv))
    gbs = vbytes / verify_s / 1e9
    k1_mean = float(np.mean(k1))
    k1_gbs = vbytes / k1_mean / 1e9
    kr_gbs = vbytes / kr_mean / 1e9

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
            "prompt_workload": wp.name if pbufs else None,
            "parallelism": "single-gpu",
        },
        "verify": {
            "us_per_call": round(verify_s * 1e6, 3),
            "kernel_us": round(k1_mean * 1e6, 3),
            "reduce_us": round(float(np.mean(kr)) * 1e6, 3),
            "kv_bytes": vbytes,
            "unique_kv_bytes": wv.unique_kv_bytes(),
            "partial_bytes": ops.workspace_bytes(wv.n_rows, wv.n_q_heads, wv.head_dim, S),
            "gbs": round(gbs, 2),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "kernel_gbs": round(k1_gbs, 2),
            "kernel_frac_hbm": round(k1_gbs / HBM_PEAK_GBS, 4),
            "kernel_us_back_to_back": round(kr_mean * 1e6, 3),
            "reduce_us_back_to_back": round(rr_mean * 1e6, 3),
            "call_us_back_to_back": round(cr_mean * 1e6, 3),
            "launches_back_to_back": KR,
        },
        "roofline": {
            "kernel": kernel_of_path(verify_path),
            "bound": "hbm",
            "achieved": round(kr_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kr_gbs / HBM_PEAK_GBS, 4),
            "launch_us": round(kr_mean * 1e6, 3),
            "traffic": load_traffic("verify"),
        },
    }
    if pbufs:
        flops = wp.algorithmic_flops()
        issued = issued_mfma_flops(wp, prompt_path)
        kp_mean = float(np.mean(kp))
        tf = flops / kp_mean / 1e12
        tfi = issued / kp_mean / 1e12
        res["prompt"] = {
            "workload": wp.name,
            "config": W.describe(wp),
            "path": prompt_path,
            "ms_per_call": round(kp_mean * 1e3, 4),
            "algorithmic_flop": flops,
            "issued_mfma_flop": issued,
            "tflops": round(tf, 2),
            "frac_mfma": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "issued_tflops": round(tfi, 2),
            "frac_mfma_issued": round(tfi / FP16_MFMA_PEAK_TFLOPS, 4),
            "rotating_copies": len(pbufs),
        }
        res["prompt_roofline"] = {
            "kernel": kernel_of_path(prompt_path),
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "frac_issued": round(tfi / FP16_MFMA_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prompt"),
        }
    res["host_wall_s"] = round(wall, 3)
    ceil = read_ceiling(ops, dev)
    res["read_ceiling"] = ceil
    res["verify"]["frac_of_read_ceiling"] = round(gbs / ceil["gbs"], 4)
    res["verify"]["kernel_frac_of_read_ceiling"] = round(k1_gbs / ceil["gbs"], 4)
    if not args.no_extra_verify:
        res["verify_configs"] = time_verify_configs(ops, dev, args, min(K, 30), hold)
    if not args.no_append:
        res["kv_append"] = time_append(ops, dev, min(K, 20), args.warmup, hold)
        res["verify_head"] = time_head(ops, dev, min(K, 20), args.warmup, hold)
        res.update(time_f16kv(ops, dev, wv, wp, min(K, 20), args.warmup, not args.no_prompt, hold))

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wv, iv)

    print(json.dumps(res), flush=True)


class Hold:
    """Keeps the GPU busy while launches are being queued: plain reads of a
    1 GiB buffer (about 0.17 ms each on this part), so that the timed launches
    find the queue ahead of them without the clocks dropping as they would
    behind an idle wait."""

    def __init__(self, ops, dev, nbytes=1 << 30):
        import torch

        self.ops = ops
        self.buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        self.sink = torch.empty(ops.STREAM_SINK_WORDS, dtype=torch.int32, device=dev)

    def __call__(self, seconds):
        for _ in range(max(1, int(seconds / 0.15e-3) + 1)):
            self.ops.stream_read(self.buf, self.sink)


def timed_calls(call, steps, warmup, hold, per_call_host_s=60e-6, marks=2):
    """Warm-up calls back to back, then `steps` timed calls, all queued behind a
    busy hold long enough for the host to queue them; returns the events
    (marks per call) after synchronising.  call(i, events) records its own
    events."""
    import torch

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [[E() for _ in range(marks)] for _ in range(steps)]
    torch.cuda.synchronize()
    hold(per_call_host_s * (warmup + steps) + 1e-3)
    for i in range(warmup):
        call(i, None)
    for i in range(steps):
        call(i + 1, ev[i])
    torch.cuda.synchronize()
    return ev


def rotating_copies(host_arrays, dev, min_bytes, cap=512):
    """Device copies of one workload's inputs, enough of them that at least
    min_bytes cycle (each copy holds every input array)."""
    import torch

    per = sum(a.nbytes for a in host_arrays)
    n = max(1, min(cap, -(-int(min_bytes) // max(per, 1))))
    base = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in host_arrays]
    return [base] + [[t.clone() for t in base] for _ in range(n - 1)]


def rows_per_group_of(path, default):
    m = re.search(r"rows_per_group(\d+)", path or "")
    return int(m.group(1)) if m else default


def kernel_of_path(path):
    """The attention kernel instance a launch description names."""
    if not path:
        return None
    kv16 = "kvf16" in path
    hd = re.search(r"hd(\d+)", path).group(1)
    qf32 = "qf32" in path
    nq = re.search(r"tiles(\d+)", path).group(1)
    final = path.startswith("prompt")
    b = lambda x: "true" if x else "false"  # noqa: E731
    if " own" in path:
        name = "attend_own_f16kv_kernel" if kv16 else "attend_own_q8_kernel"
        return f"{name}<{hd}, {b(qf32)}, {b(final)}, {nq}>"
    name = "attend_f16kv_kernel" if kv16 else "attend_q8_kernel"
    return f"{name}<{hd}, {b(qf32)}, {b(final)}, {nq}>"


def issued_mfma_flops(w, path):
    """FLOPs of the 16x16x32 f16 MFMAs (16,384 each) the attention kernel issues
    for workload w in the launch `path` describes: per (16-vector tile, 32-key
    tile) QK takes head_dim/32 blocks x 2 key subtiles (x2 for fp32 q: hi and
    lo), PV head_dim/16 output tiles x 3 terms (Vhi Phi, Vlo Phi, Vhi Plo; two
    over an fp16 cache).  Each row group scans keys 0 .. its last row's
    position, in whole 32-key tiles."""
    hd = w.head_dim
    qf32 = "qf32" in path
    kv16 = "kvf16" in path
    rg = rows_per_group_of(path, 1)
    per_pair = (hd // 32) * 2 * (2 if qf32 else 1) + (hd // 16) * (2 if kv16 else 3)
    if w.kind == "prompt":
        n, p0 = w.n_queries, w.pos0
    else:
        n, p0 = w.n_rows, w.ctx_len
    total = 0
    for r0 in range(0, n, rg):
        nr = min(rg, n - r0)
        vtiles = -(-nr * w.group // 16)
        ktiles = -(-(p0 + r0 + nr) // 32)
        total += vtiles * ktiles
    return total * w.n_kv_heads * per_pair * 16384


# The verify configurations reported beside the headline: (workload, rows_per_group,
# label); rows_per_group 0 = the library's own grouping.
EXTRA_VERIFY = [("verify_window", 0, "verify_window"), ("verify_batch", 4, "verify_batch_r4"),
                ("verify_batch", 0, "verify_batch_auto"), ("verify_batch", 32, "verify_batch_r32"),
                ("tiny_verify", 0, "tiny_verify")]


def time_verify_configs(ops, dev, args, steps, hold):
    """The other verify workloads: whole call and attention kernel alone (HIP
    events, rotating copies of >= rotate_bytes), KV bytes per pass over the row
    groups and unique, and the partials' bytes."""
    import torch

    import workloads as W

    out = {}
    cache = {}
    for name, rg, label in EXTRA_VERIFY:
        w = W.WORKLOADS[name]
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            inp = W.generate(w)
            cache[name] = rotating_copies([inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales],
                                          dev, args.rotate_bytes)
        bufs = cache[name]
        k1, k2, tot, S, path, kb, rb = time_verify(ops, bufs, w, rg, steps, args.warmup, hold)
        rg_used = rows_per_group_of(path, rg or w.rows_per_group)
        per_pass = w.visible_kv_bytes(rg_used)
        uniq = w.unique_kv_bytes()
        out[label] = {
            "workload": name,
            "rows_per_group": rg_used,
            "splits": S,
            "path": path,
            "kernel": kernel_of_path(path),
            "us_per_call": round(tot * 1e6, 3),
            "kernel_us": round(k1 * 1e6, 3),
            "reduce_us": round(k2 * 1e6, 3),
            "kernel_us_back_to_back": round(kb * 1e6, 3),
            "reduce_us_back_to_back": round(rb * 1e6, 3),
            "kv_bytes_per_pass": per_pass,
            "unique_kv_bytes": uniq,
            "partial_bytes": ops.workspace_bytes(w.n_rows, w.n_q_heads, w.head_dim, S),
            "gbs_per_pass": round(per_pass / tot / 1e9, 2),
            "gbs_unique": round(uniq / tot / 1e9, 2),
            "frac_hbm_per_pass": round(per_pass / tot / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_gbs_per_pass": round(per_pass / k1 / 1e9, 2),
            "kernel_frac_hbm_per_pass": round(per_pass / k1 / 1e9 / HBM_PEAK_GBS, 4),
            "rotating_copies": len(bufs),
            "steps": steps,
        }
    cache.clear()
    torch.cuda.empty_cache()
    return out


def summarize_trace(path, skip_first, tail=0):
    """Per-kernel durations from a rocprofv3 kernel-trace CSV: launches grouped by
    (kernel, grid), the first skip_first of each group dropped (or, with tail,
    only the last `tail` kept); markdown table."""
    import csv
    import statistics

    groups = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Kind") != "KERNEL_DISPATCH":
                continue
            key = (row["Kernel_Name"], (row["Grid_Size_X"], row["Grid_Size_Y"], row["Grid_Size_Z"]),
                   row["Workgroup_Size_X"])
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3  # us
            groups.setdefault(key, []).append((int(row["Dispatch_Id"]), dur))
    print(f"| kernel | grid (threads) | block | launches used (of all) | median (us) | mean (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|---|---|")
    rows = []
    for (name, grid, block), d in groups.items():
        d.sort()
        used = [x for _, x in (d[-tail:] if tail else d[skip_first:])] or [x for _, x in d]
        rows.append((statistics.median(used) * len(used), name, grid, block, used, len(d)))
    for _, name, grid, block, used, n_all in sorted(rows, reverse=True):
        short = name if len(name) <= 110 else name[:107] + "..."
        print(f"| `{short}` | {'x'.join(grid)} | {block} | {len(used)} ({n_all}) | "
              f"{statistics.median(used):.2f} | {statistics.mean(used):.2f} | {min(used):.2f} | {max(used):.2f} |")


def _pmc_rows(paths):
    """(kernel, grid threads, counter) -> per-dispatch values, from rocprofv3
    counter-collection CSVs (files, or directories searched for them)."""
    import csv
    import glob

    files = []
    for p in paths:
        files += sorted(glob.glob(os.path.join(p, "**", "*counter_collection.csv"), recursive=True)) \
            if os.path.isdir(p) else [p]
    out = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"], int(row["Grid_Size"]), row["Counter_Name"])
                out.setdefault(key, []).append(float(row["Counter_Value"]))
    return out


def _short_kernel(name):
    m = re.match(r"(?:void )?(?:attnq8::)?([^(]+)", name)
    return m.group(1) if m else name


def summarize_pmc(paths):
    rows = _pmc_rows(paths)
    counters = sorted({c for _, _, c in rows})
    kernels = sorted({(k, g) for k, g, _ in rows}, key=lambda x: (x[0], x[1]))
    print("| kernel | grid (threads) | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|---|" + "---|" * len(counters))
    for k, g in kernels:
        vals = [rows.get((k, g, c)) for c in counters]
        n = max(len(v) for v in vals if v)
        cells = [f"{np.mean(v):,.4g}" if v else "" for v in vals]
        print(f"| `{_short_kernel(k)}` | {g:,} | {n} | " + " | ".join(cells) + " |")


# traffic.json keys: the kernels bench.py reports `traffic` for (the long
# verify's reducer is the reduce_partials_kernel<256> launch with the smallest
# grid among the configurations bench.py times)
TRAFFIC_KEYS = {
    "verify": "attend_q8_kernel<256, true, false, 2>",
    "verify_window": "attend_q8_kernel<256, true, false, 3>",
    "prompt": "attend_own_q8_kernel<256, false, true, 6>",
    "reduce": "reduce_partials_kernel<256>",
    "append": "kv_append_q8_kernel<true>",
    "head": "head_greedy_kernel",
    "verify_f16kv": "attend_f16kv_kernel<256, true, false, 2>",
    "prompt_f16kv": "attend_own_f16kv_kernel<256, false, true, 6>",
}


def traffic_from(d, write):
    fetch = _pmc_rows([os.path.join(d, "FETCH_SIZE")])
    write_rows = _pmc_rows([os.path.join(d, "WRITE_SIZE")])
    fetch_c = _pmc_rows([os.path.join(d, "FETCH_SIZE_copy")])
    write_c = _pmc_rows([os.path.join(d, "WRITE_SIZE_copy")])

    def copy_kib(rows, counter):
        # the device copy of COPY_BYTES: the largest per-dispatch value of the counter
        vals = [np.mean(v) for (k, g, c), v in rows.items() if c == counter]
        return max(vals)

    kib = COPY_BYTES / 1024
    ff = kib / copy_kib(fetch_c, "FETCH_SIZE")
    wf = kib / copy_kib(write_c, "WRITE_SIZE")
    print(f"copy calibration: {COPY_BYTES:,} bytes read and written; FETCH_SIZE factor {ff:.3f}, "
          f"WRITE_SIZE factor {wf:.3f}")
    print("| key | kernel | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |")
    print("|---|---|---|---|---|---|---|")
    kernels = {}
    for key, short in TRAFFIC_KEYS.items():
        cands = sorted({g for (k, g, c) in fetch if _short_kernel(k) == short and c == "FETCH_SIZE"})
        if not cands:
            continue
        g = cands[0]
        name = next(k for (k, gg, c) in fetch if _short_kernel(k) == short and gg == g)
        fr = float(np.mean(fetch[(name, g, "FETCH_SIZE")]))
        wr = float(np.mean(write_rows.get((name, g, "WRITE_SIZE"), [float("nan")])))
        rb, wb = fr * 1024 * ff, wr * 1024 * wf
        kernels[key] = {"read_bytes": int(rb), "write_bytes": int(wb), "total_bytes": int(rb + wb)}
        print(f"| {key} | `{short}` | {g:,} | {fr:,.1f} | {wr:,.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
    if write:
        with open(TRAFFIC_FILE, "w") as f:
            json.dump({"source_hash": kernel_source_hash(), "fetch_factor": round(ff, 4),
                       "write_factor": round(wf, 4), "kernels": kernels}, f, indent=1)
            f.write("\n")
        print(f"wrote {TRAFFIC_FILE} (sources {kernel_source_hash()})")


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


def time_append(ops, dev, steps, warmup, hold):
    import torch

    T, H, hd = APPEND_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rows = [[torch.randn((T, H, hd), generator=g, device=dev) for _ in range(2)] for _ in range(2)]
    kc = torch.empty((H, T, hd), dtype=torch.int8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((H, T, hd // 32), dtype=torch.float16, device=dev)
    vs = torch.empty_like(ks)

    def call(i, e):
        k, v = rows[i % 2]
        if e:
            e[0].record()
        ops.kv_append(k, kc, ks, 0, v, vc, vs)
        if e:
            e[1].record()

    call(0, None)
    path = ops.last_path()
    ev = timed_calls(call, steps, warmup, hold)
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


def _events_mean(call, steps, warmup, hold):
    """Mean duration (s) of call(i) over `steps` timed calls (timed_calls)."""

    def c(i, e):
        if e:
            e[0].record()
        call(i)
        if e:
            e[1].record()

    ev = timed_calls(c, steps, warmup, hold)
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3


def time_f16kv(ops, dev, wv, wp, steps, warmup, with_prompt, hold):
    """The verify and prompt workloads over an fp16 K/V cache (the same seeded
    draws rounded to fp16 instead of quantised), measured beside the int8 path."""
    import torch

    import workloads as W

    out = {}
    iv = W.generate_f16kv(wv)
    copies = rotating_copies([iv.q, iv.k, iv.v], dev, 1.1e9)
    S = ops.verify_splits(wv.n_q_heads, wv.n_kv_heads, wv.head_dim, wv.ctx_len, wv.n_rows, 0)
    ws = torch.empty(ops.workspace_bytes(wv.n_rows, wv.n_q_heads, wv.head_dim, S),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((wv.n_rows, wv.n_q_heads, wv.head_dim), dtype=torch.float32, device=dev)

    def vcall(i):
        q, k, v = copies[i % len(copies)]
        ops.verify_f16kv_partials(q, k, v, ctx_len=wv.ctx_len, n_splits=S, workspace=ws)

    vcall(0)
    vpath = ops.last_path()
    t = _events_mean(vcall, steps, warmup, hold)
    # fp16 K and V bytes of the grouping the library chose
    rg = rows_per_group_of(vpath, wv.rows_per_group)
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
    del copies
    torch.cuda.empty_cache()
    if with_prompt:
        ip = W.generate_f16kv(wp)
        pout = torch.empty((wp.n_queries, wp.n_q_heads, wp.head_dim), dtype=torch.float32,
                           device=dev)
        pcopies = rotating_copies([ip.q, ip.k, ip.v], dev, 1.1e9)

        def pcall(i):
            q, k, v = pcopies[i % len(pcopies)]
            ops.prompt_f16kv(q, k, v, q_pos0=wp.pos0, kv_len=wp.kv_len, out=pout)

        pcall(0)
        ppath = ops.last_path()
        tp = _events_mean(pcall, max(3, steps // 4), max(3, warmup // 4), hold)
        tf = wp.algorithmic_flops() / tp / 1e12
        tfi = issued_mfma_flops(wp, ppath) / tp / 1e12
        out["prompt_f16kv"] = {
            "workload": f"{wp.name} over an fp16 cache",
            "path": ppath,
            "ms_per_call": round(tp * 1e3, 4),
            "tflops": round(tf, 2),
            "frac_mfma": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "frac_mfma_issued": round(tfi / FP16_MFMA_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prompt_f16kv"),
        }
    return out


# The verify head measured beside the attention: greedy token and top
# probability of 5 rows of 248,320 fp32 logits (the sampler page's benchmark
# shape), several rotating copies so that the rows come from HBM.
HEAD_SHAPE = (5, 248320)


def time_head(ops, dev, steps, warmup, hold):
    import torch

    rows, V = HEAD_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    copies = [torch.randn((rows, V), generator=g, device=dev) * 3 for _ in range(64)]
    ws = torch.zeros(ops.head_workspace_bytes(rows, V), dtype=torch.uint8, device=dev)
    tok = torch.empty(rows, dtype=torch.int32, device=dev)
    top = torch.empty(rows, dtype=torch.float32, device=dev)

    def call(i, e):
        if e:
            e[0].record()
        ops.verify_head_greedy(copies[i % len(copies)], workspace=ws, token=tok, top_prob=top)
        if e:
            e[1].record()

    call(0, None)
    path = ops.last_path()
    ev = timed_calls(call, steps, warmup, hold)
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    # the same calls back to back (events around the region, divided by its
    # launches): no per-call event latency
    n_b2b = max(steps, 10)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold(60e-6 * n_b2b + 1e-3)
    r0.record()
    for i in range(n_b2b):
        call(i + 1, None)
    r1.record()
    torch.cuda.synchronize()
    tb = r0.elapsed_time(r1) / n_b2b * 1e-3
    moved = rows * V * 4
    return {
        "workload": f"{rows} rows x {V} fp32 logits: greedy token + top probability",
        "path": path,
        "us_per_call": round(t * 1e6, 3),
        "us_per_call_back_to_back": round(tb * 1e6, 3),
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


def time_verify(ops, bufs, w, rows_per_group, steps, warmup, hold):
    """Mean durations (s) over rotating inputs: the attention kernel alone and the
    reducer after it (with the launch gap before it), both from the steps that
    record an event between the two, the whole call from the steps that do
    not, and each kernel launched back to back (per launch)."""
    import torch

    S = ops.verify_splits(w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_len, w.n_rows,
                          rows_per_group)
    ws = torch.empty(ops.workspace_bytes(w.n_rows, w.n_q_heads, w.head_dim, S),
                     dtype=torch.uint8, device=bufs[0][0].device)
    out = torch.empty((w.n_rows, w.n_q_heads, w.head_dim), dtype=torch.float32,
                      device=ws.device)

    paths = []

    # (as in the main run: the kernel alone on odd steps, the whole call on even ones)
    def call(i, e):
        q, kc, ks, vc, vs = bufs[i % len(bufs)]
        if e:
            e[0].record()
        ops.verify_partials(q, kc, ks, vc, vs, ctx_len=w.ctx_len,
                            rows_per_group=rows_per_group, n_splits=S, workspace=ws)
        if not paths:
            paths.append(ops.last_path())
        if e and (i % 2 == 0 or steps < 2):
            e[1].record()
        ops.reduce_partials(ws, w.n_rows, w.n_q_heads, w.head_dim, S, out=out)
        if e:
            e[2].record()

    call(0, None)
    path = paths[0]
    ev = timed_calls(call, steps, warmup, hold, marks=3)
    odd = [e for i, e in enumerate(ev) if i % 2 == 1 or steps < 2]
    even = [e for i, e in enumerate(ev) if i % 2 == 0]
    k1 = float(np.mean([e[0].elapsed_time(e[1]) for e in odd])) * 1e-3
    call = float(np.mean([e[0].elapsed_time(e[2]) for e in even])) * 1e-3
    k2 = float(np.mean([e[1].elapsed_time(e[2]) for e in odd])) * 1e-3
    # each kernel alone, launched back to back (events around the region)
    R = max(steps, 10)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    regions = []
    for part in ("kernel", "reduce"):
        torch.cuda.synchronize()
        hold(60e-6 * R + 1e-3)
        r0.record()
        for i in range(R):
            if part == "kernel":
                q, kc, ks, vc, vs = bufs[(i + 1) % len(bufs)]
                ops.verify_partials(q, kc, ks, vc, vs, ctx_len=w.ctx_len,
                                    rows_per_group=rows_per_group, n_splits=S, workspace=ws)
            else:
                ops.reduce_partials(ws, w.n_rows, w.n_q_heads, w.head_dim, S, out=out)
        r1.record()
        torch.cuda.synchronize()
        regions.append(r0.elapsed_time(r1) / R * 1e-3)
    return k1, k2, call, S, path, regions[0], regions[1]


def sweep(args):
    import torch

    import workloads as W
    from attention_int8_quantized_amd import ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = min(args.steps, 30)
    hold = Hold(ops, dev)
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
            cells[rg] = time_verify(ops, bufs, w, rg, steps, args.warmup, hold)
        t1 = cells[1][2]
        for rg in SWEEP_GROUPS:
            k1, k2, tot, S, path = cells[rg][:5]
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
