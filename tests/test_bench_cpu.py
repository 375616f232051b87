"""bench.py's host-side contract (no GPU needed)."""

import json
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_keyed_to_the_sources(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert {"verify", "prompt", "reduce"} <= set(t["kernels"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: t["source_hash"])
    v = bench.load_traffic("verify")
    assert v["read_bytes"] > 0 and v["write_bytes"] > 0
    assert v["total_bytes"] == v["read_bytes"] + v["write_bytes"]
    assert bench.load_traffic("no such kernel") is None
    # counters taken on other sources are not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("verify") is None


def test_source_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    import shutil

    csrc = tmp_path / "attention_int8_quantized_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "attention_int8_quantized_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = csrc / "attend_kernel.h"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("namespace attnq8 {", "namespace attnq8 {  /* x */", 1))
    assert bench.kernel_source_hash() == h0
    f.write_text(text.replace("kRescaleSlack = 15.0f", "kRescaleSlack = 14.0f", 1))
    assert bench.kernel_source_hash() != h0


def test_strip_comments_keeps_literals():
    src = 'a = 1; // gone "x"\n/* gone\n */ s = "k // not /* a */ comment"; c = \'"\';'
    assert bench.strip_comments(src) == 'a = 1; s = "k // not /* a */ comment"; c = \'"\';'


def test_issued_mfma_flops_and_kernel_names():
    import workloads as W

    p = "prompt kvq8 hd256 qf16 tiles6 own rows_per_group8 groups256 kv_heads1"
    assert bench.kernel_of_path(p) == "attend_own_q8_kernel<256, false, true, 6>"
    o = "verify kvq8 hd128 qf32 tiles8 own rows_per_group32 groups1 splits32 kv_heads8"
    assert bench.kernel_of_path(o) == "attend_own_q8_kernel<128, true, false, 8>"
    # fp16 q: 16 QK + 48 PV MFMAs per (16 vectors, 32 keys) = 2,048 FLOP per pair,
    # twice the algorithmic 4 * 256 = 1,024, plus the masked halves of diagonal tiles
    r = bench.issued_mfma_flops(W.PROMPT_CHUNK, p) / W.PROMPT_CHUNK.algorithmic_flops()
    assert 2.0 < r < 2.01
    v = "verify kvq8 hd256 qf32 tiles2 rows_per_group4 groups1 splits64 kv_heads4"
    assert bench.kernel_of_path(v) == "attend_q8_kernel<256, true, false, 2>"
    # fp32 q: 32 + 48 MFMAs per pair of tiles, 24 of 32 vector slots used
    r = bench.issued_mfma_flops(W.LONG_VERIFY, v) / W.LONG_VERIFY.algorithmic_flops()
    assert abs(r - 80 * 16384 / 512 / 1024 * 32 / 24) < 1e-3


def test_trace_summary_drops_the_first_launches(tmp_path, capsys):
    head = ('"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp",'
            '"Workgroup_Size_X","Grid_Size_X","Grid_Size_Y","Grid_Size_Z"\n')
    rows = [f'"KERNEL_DISPATCH",{i},"k",{1000 * i},{1000 * i + (9000 if i < 2 else 2000)},512,1024,1,1\n'
            for i in range(6)]
    f = tmp_path / "t_kernel_trace.csv"
    f.write_text(head + "".join(rows))
    bench.summarize_trace(str(f), 2)
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("| `k`")][0]
    assert "| 4 (6) | 2.00 | 2.00 | 2.00 | 2.00 |" in line
