"""CPU tests of the benchmark's host arithmetic: the algorithmic FLOP and
byte counts its roofline figures divide by, checked against closed forms
worked out by hand for the measured workloads (pairs per head: T(T+1)/2 for
a full-causal layer, W(W+1)/2 + (T-W)W for a W-key window; 640 FLOP per pair
and head; 73,856 bytes per token of the prefill; 10,240 bytes per visible
cached token plus 63,616 bytes per sequence of the decode), and its refusal
of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_flops():
    flops = lambda B, T, W, P=0: bench.pairs_prefill(B, T, W, P) * bench.N_HEADS * bench.FLOP_PER_PAIR
    assert flops(1, 4096, 0) == 4096 * 4097 // 2 * 80 * 640 == 429_601_587_200
    assert flops(2, 32768, 128) == 2 * (128 * 129 // 2 + (32768 - 128) * 128) * 80 * 640 == 428_664_422_400
    assert flops(1, 131072, 0) == 439_808_006_553_600
    assert flops(1, 256, 0) * 5 // 80 == 105_267_200                 # the tiny config's 5 heads
    # prefix: the rows after P only
    assert bench.pairs_prefill(1, 32768, 0, 28672) == 32768 * 32769 // 2 - 28672 * 28673 // 2
    assert bench.pairs_prefill(1, 100, 1000) == bench.pairs_prefill(1, 100, 0)   # window >= T


def test_prefill_bytes():
    assert bench.prefill_bytes(1, 4096) == 4096 * 73_856 == 302_514_176
    assert bench.prefill_bytes(2, 32768) == 4_840_226_816
    assert bench.prefill_bytes(1, 131072) == 9_680_453_632
    # prefix: K/V of every row, the query side of the new rows only
    per_kv = 16 * (192 + 128) * 2
    assert bench.prefill_bytes(1, 200, prefix=100) == 100 * (73_856 - per_kv) + 200 * per_kv


def test_decode_bytes():
    lengths = [8192, 65536, 100]
    assert bench.decode_bytes(lengths, 0) == 10_240 * sum(lengths) + 3 * 63_616 + 4 * 4
    assert bench.decode_bytes(lengths, 128) == 10_240 * (128 + 128 + 100) + 3 * 63_616 + 4 * 4


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_results_log_appends_and_resumes(tmp_path, monkeypatch):
    """--results: one JSON record per configuration; --resume skips the ones
    already recorded for the same commit, and only those."""
    import json
    path = str(tmp_path / "results.jsonl")
    monkeypatch.setattr(bench, "git_sha", lambda: "abc")
    r = bench.Results(path, resume=True)
    assert not r.skip("pf_full_4k")
    r.add("pf_full_4k", {"time_ms": 0.37, "mfma_frac": 0.46})
    r.add("dec_full", {"time_ms": 4.3})
    rows = [json.loads(x) for x in open(path)]
    assert [x["config"] for x in rows] == ["pf_full_4k", "dec_full"]
    assert rows[0]["git_sha"] == "abc" and rows[0]["seed"] == 0 and rows[0]["time_ms"] == 0.37
    assert "host_cpus" in rows[0] and "cpu_model" in rows[0]
    again = bench.Results(path, resume=True)
    assert again.skip("pf_full_4k") and again.skip("dec_full") and not again.skip("pf_swa_32k")
    assert not bench.Results(path, resume=False).skip("pf_full_4k")
    monkeypatch.setattr(bench, "git_sha", lambda: "def")           # another commit: nothing is skipped
    assert not bench.Results(path, resume=True).skip("pf_full_4k")
    bench.Results(None, resume=False).add("x", {})                 # no file: a no-op


def test_traffic_records_survive_comment_edits(tmp_path, monkeypatch):
    """A traffic record holds while the kernels' code is unchanged: the source
    hash ignores comments and spacing, and changes with the code."""
    import shutil
    src = os.path.join(ROOT, "attention_gdla_prefill_amd", "csrc")
    dst = tmp_path / "attention_gdla_prefill_amd" / "csrc"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.o", "*.so"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash("prefill")
    f = dst / "prefill_gfx950.hip"
    text = f.read_text()
    f.write_text("// a new first line\n" + text.replace("namespace gdla {", "namespace gdla {  /* x */\n\n", 1))
    assert bench.source_hash("prefill") == h0
    f.write_text(text.replace("constexpr int BM = 64;", "constexpr int BM = 32;", 1))
    assert bench.source_hash("prefill") != h0
    assert bench.strip_comments('a = "//"; // c\nb = 1; /* d */ c') == 'a = "//"; b = 1; c'
