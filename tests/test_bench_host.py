"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline fraction, the HBM-traffic summary built from rocprofv3 counter CSVs,
the check that ties a summary to the kernel sources it was taken on, and the
refusal of multi-GPU runs.

The byte counts are pinned to totals derived another way: per matrix or per
chunk, enumerated chunk by chunk, or summed from the tensors one by one.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_solver_bytes_per_matrix():
    # 16 x 512 tokens, 64 heads, f32 in and out: 8192 64x64 matrices, each
    # read once as A and written once as X
    cfg = synth.CONFIGS["packed_16x512_h64_f32"]
    lengths = synth.config_lengths(cfg)
    mats = sum(-(-n // 64) for n in lengths) * cfg["H"]
    assert mats == 8192
    assert bench.algorithmic_bytes(lengths, cfg["H"], 4, 4) == mats * 2 * 64 * 64 * 4 == 268435456


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_solver_bytes_ragged_chunk_by_chunk(chunk):
    # 48 ragged requests (partial last chunks): count the rows of every chunk
    # of every request; each row holds `chunk` entries of A (f32) and of X (bf16)
    cfg = synth.CONFIGS["packed_ragged48_h64_f32_bf16"]
    lengths = synth.config_lengths(cfg)
    assert sum(lengths) == 33139
    rows = 0
    for n in lengths:
        start = 0
        while start < n:
            rows += min(chunk, n - start)
            start += chunk
    assert bench.algorithmic_bytes(lengths, cfg["H"], 4, 2, C=chunk) == rows * cfg["H"] * chunk * 6


def test_kkt_bytes_per_chunk_head():
    # one full chunk-head with K = 128, bf16 keys and write strengths, f32
    # decays and f32 X: 64 rows x (256 B keys + 512 B decays + 2 B beta +
    # 256 B of X) = 65,664 B
    per_chunk_head = 64 * (128 * 2) + 64 * (128 * 4) + 64 * 2 + 64 * 64 * 4
    assert per_chunk_head == 65664
    assert bench.kkt_algorithmic_bytes([512] * 16, 64, 128, 2, 4) == 8192 * per_chunk_head
    # f32 keys and write strengths
    per_f32 = 64 * (128 * 4) + 64 * (128 * 4) + 64 * 4 + 64 * 64 * 4
    assert bench.kkt_algorithmic_bytes([512] * 16, 64, 128, 4, 4) == 8192 * per_f32 == 673185792


def test_decode_bytes_tensor_by_tensor():
    # one decode step, B = 32 sequences, 32 heads of 128, conv width 4, bf16
    # activations: every tensor the step touches, listed one by one
    B, H, d, W = 32, 32, 128, 4
    pairs = B * H
    tensors = {
        "state read": pairs * d * d * 4,
        "state written": pairs * d * d * 4,
        "conv windows read (q, k, v)": pairs * 3 * (W - 1) * d * 4,
        "conv windows written": pairs * 3 * (W - 1) * d * 4,
        "q, k, v in": pairs * 3 * d * 2,
        "output gate z": pairs * d * 2,
        "decays (f32)": pairs * d * 4,
        "write strength (f32)": pairs * 4,
        "output": pairs * d * 2,
        "conv taps (q, k, v)": H * 3 * W * d * 4,
        "norm weights": d * 4,
    }
    assert sum(tensors.values()) == 145691136
    assert bench.decode_algorithmic_bytes(B, H, d, W, 2, 2) == 145691136
    # padding entries move nothing of their own
    assert (bench.decode_algorithmic_bytes(B, H, d, W, 2, 2, padding=5) ==
            145691136 - 5 * H * (tensors["state read"] + tensors["state written"] +
                                 tensors["conv windows read (q, k, v)"] +
                                 tensors["conv windows written"] + tensors["q, k, v in"] +
                                 tensors["output gate z"] + tensors["decays (f32)"] +
                                 tensors["write strength (f32)"] + tensors["output"]) // pairs)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))
    return str(path)


def test_record_traffic_scales_by_the_copy(tmp_path):
    # The copy probe moves A's byte count each way; its FETCH_SIZE reads twice
    # that and its WRITE_SIZE exactly that, so the kernel's FETCH_SIZE is
    # halved and its WRITE_SIZE kept. Dispatches of other kernels are ignored.
    w = "packed_16x512_h64_f32"
    known_kib = bench.copy_bytes_of(w) / 1024
    assert known_kib == 131072
    k = "void kda::tril_inv_fused_mfma<kda::F32, kda::F32, false>(kda::Problem)"
    fetch = _counter_csv(tmp_path / "f.csv", [(k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 1200.0),
                                              ("other_kernel", "FETCH_SIZE", 9e9)])
    write = _counter_csv(tmp_path / "w.csv", [(k, "WRITE_SIZE", 2048.0)])
    cfetch = _counter_csv(tmp_path / "cf.csv",
                          [("kda_probe_copy_kernel(float4 const*, float4*, long)", "FETCH_SIZE",
                            2 * known_kib)])
    cwrite = _counter_csv(tmp_path / "cw.csv",
                          [("kda_probe_copy_kernel(float4 const*, float4*, long)", "WRITE_SIZE",
                            known_kib)])
    out = tmp_path / "t.json"
    t = bench.record_traffic(w, [fetch, write, cfetch, cwrite], str(out))
    assert t["dispatches"] == {"fetch": 2, "write": 1}
    assert t["fetch_scale"] == 0.5 and t["write_scale"] == 1.0
    assert t["hbm_read_bytes_per_launch"] == 1100 * 1024 * 0.5
    assert t["hbm_write_bytes_per_launch"] == 2048 * 1024
    assert t["hbm_bytes_per_launch"] == 550 * 1024 + 2048 * 1024
    assert json.loads(out.read_text()) == t


def test_traffic_summary_tied_to_kernel_sources(tmp_path, monkeypatch):
    w = "packed_16x512_h64_f32"
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda _: str(f))
    assert bench.load_traffic(w) is None  # missing
    f.write_text(json.dumps({"kernel_hash": bench.kernel_hash(w), "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic(w) == 123
    f.write_text(json.dumps({"kernel_hash": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic(w) is None  # taken on other sources


def test_kernel_hash_ignores_comments_only():
    a = "int f(int x) { return x + 1; }  // one\n/* two\n lines */ int g;"
    b = "int f(int x)\n{\n    return x + 1;  // changed comment\n}\nint g;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x + 1", "x + 2"))


def test_kernel_sources_per_workload():
    # every timed workload names the sources its kernel is built from, and
    # they exist
    for w in bench.WORKLOADS:
        pattern, files = bench.kernel_of(w)
        assert pattern and files
        for fn in files:
            assert os.path.isfile(os.path.join(ROOT, "tril_solve_amd", "csrc", fn)), fn
        assert len(bench.kernel_hash(w)) == 16


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_multi_gpu_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_line_labels_algorithmic_and_measured_rates():
    """roofline.achieved is algorithmic bytes over the kernel time and says
    so; the measured HBM rate uses the counter bytes over the same time."""
    import types
    args = types.SimpleNamespace(steps=10, warmup=1)
    k_avg = 45e-6
    out = bench.base_line(args, 10 * 46e-6, k_avg, {}, 8192, 268435456, 4, bench.METRIC, None,
                          {"workload": "w"}, "f32 A -> f32 X")
    assert out["roofline"]["bytes"] == "algorithmic"
    assert out["roofline"]["achieved"] == pytest.approx(268435456 / 45e-6 / 1e9)
    assert out["dtype"] == "f32" and out["io_dtype"] == "f32 A -> f32 X"
    assert "hbm_measured" not in bench.with_measured_hbm(dict(out), None)
    bench.with_measured_hbm(out, 235368201)
    assert out["roofline"]["traffic"] == 235368201
    m = out["hbm_measured"]
    assert m["achieved"] == pytest.approx(235368201 / 45e-6 / 1e9)
    assert m["frac"] == pytest.approx(m["achieved"] / 8000.0)


def test_kernel_patterns_match_the_kernels_each_workload_runs():
    """The counter summaries are matched to rocprofv3's demangled names: a
    workload's pattern must cover every kernel its launches can run (one-round
    and multi-round forms) and none of the other paths'."""
    import re
    names = {
        "packed_16x512_h64_f32": ["void kda::tril_inv_fused_heads4<kda::F32, kda::F32>(kda::Problem)",
                                  "void kda::tril_inv_fused_mfma<kda::F32, kda::F32, true>(kda::Problem)",
                                  "void kda::tril_inv_fused_cols<kda::F32, kda::F32, 2, 1>(kda::Problem)"],
        "packed_16x512_h64_c32_f32": ["void kda::tril_inv_c32_group<kda::F32, kda::F32>(kda::Problem)",
                                      "void kda::tril_inv_c32<kda::F32, kda::F32, true>(kda::Problem)"],
        "packed_16x512_h64_c16_f32": ["void kda::tril_inv_c16<kda::F32, kda::F32>(kda::Problem)"],
    }
    others = ["kda_probe_copy_kernel(float __vector(4) const*, float __vector(4)*, long)",
              "void kda::tril_inv_split_merge_heads4<kda::F32, kda::F32>(kda::Problem)"]
    for w, ks in names.items():
        pat = re.compile(bench.kernel_of(w)[0])
        for k in ks:
            assert pat.search(k), (w, k)
        for k in others + [n for v, l in names.items() if v != w for n in l]:
            assert not pat.search(k), (w, k)
