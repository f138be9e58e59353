"""Host-side checks of bench.py: the multi-GPU refusal, the constants behind its
roofline figures, and the counter summary it reads traffic from (no GPU)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_constants():
    # 6KV + C(3K + 2V) with C = 64, K = V = 128
    assert bench.F_ALG == 139264
    # q, k, v, g in (bf16, 128 each), beta in (bf16), out (bf16, 128)
    assert bench.BYTES_ALG == 1282
    # W, Qg, Kbar^T, U (64 x 128 fp16 each), the nonzero 3/4 of A_qk (64 x 64 fp16), exp(G_n)
    # (128 fp32) per chunk-head
    assert bench.INTER_BYTES * 64 == 70.5 * 1024


def test_intermediates_match_the_library_workspace():
    kda = pytest.importorskip("gated_delta_rule_110_amd")
    sizes = [kda.workspace_size(1, 64 * chunks, 3) for chunks in (1, 2)]
    # one more chunk of three heads adds three chunk-heads of intermediates: the workspace keeps
    # room for all 8 A_qk fragments (2 KiB more than is ever written or read), plus alignment
    per = (sizes[1] - sizes[0]) / 3
    assert bench.INTER_BYTES * 64 + 2048 <= per <= bench.INTER_BYTES * 64 + 2048 + 1024


def _write_counter_csv(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": "C", "Counter_Value": value})


def test_traffic_summary_scaling_and_staleness(tmp_path, monkeypatch):
    pmc = tmp_path / "pmc"
    chain = "(anonymous namespace)::kda_chain_kernel(kda::ChainArgs)"
    intra = "(anonymous namespace)::kda_intra_kernel(kda::IntraArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # the copy of 1 MiB reads 512 KiB on FETCH_SIZE (scale 2) and 1024 KiB on WRITE_SIZE (scale 1)
    _write_counter_csv(str(pmc / "calf"), [(copy, 512.0), (copy, 512.0)])
    _write_counter_csv(str(pmc / "calw"), [(copy, 1024.0)])
    # two dispatches per kernel: the per-dispatch mean is what counts
    _write_counter_csv(str(pmc / "fetch"), [(intra, 100.0), (intra, 300.0), (chain, 50.0), (chain, 50.0)])
    _write_counter_csv(str(pmc / "write"), [(intra, 10.0), (intra, 30.0), (chain, 5.0), (chain, 5.0)])
    (pmc / "calibration_bytes.txt").write_text(str(1 << 20))
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda name: str(out))
    res = bench.write_traffic(str(pmc), "wl")
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    assert res["kernels"]["kda_intra_kernel"] == {"read_bytes": 200 * 2 * 1024, "write_bytes": 20 * 1024,
                                                  "bytes": 420 * 1024,
                                                  "source_sha256": bench.source_digest("kda_intra_kernel")}
    assert res["kernels"]["kda_chain_kernel"]["bytes"] == (100 + 5) * 1024
    saved = json.loads(out.read_text())
    assert saved["source_sha256"] == bench.source_digest()
    assert saved["kernels"]["kda_chain_kernel"]["source_sha256"] == bench.source_digest("kda_chain_kernel")
    assert bench.load_traffic("wl", "kda_chain_kernel") == 105 * 1024
    assert bench.load_traffic("wl", "kda_chunk_table_kernel") is None
    # a kernel's summary is not used once that kernel's sources change; the others' still are
    real = bench.source_digest
    monkeypatch.setattr(bench, "source_digest",
                        lambda kernel=None: "0" * 64 if kernel == "kda_chain_kernel" else real(kernel))
    assert bench.load_traffic("wl", "kda_chain_kernel") is None
    assert bench.load_traffic("wl", "kda_intra_kernel") == 420 * 1024


def test_kernel_digests_cover_their_sources():
    # each kernel's digest changes with its own source and the shared files, and only with those
    for k, files in bench.KERNEL_SOURCES.items():
        assert "kda_common.h" in bench._COMMON_SOURCES and files
    assert bench.source_digest("kda_intra_kernel") != bench.source_digest("kda_chain_kernel")
    assert bench.source_digest("kda_chain_kernel") == bench.source_digest("kda_chain_x2_kernel")
    assert bench.source_digest("split_chain") != bench.source_digest("kda_chain_kernel")


def test_digest_ignores_comments_only():
    code = "int f(int x) {  // add one\n  return x + 1; /* done */ }\n"
    assert bench._code_only("a.hip", code) == bench._code_only("a.hip", code.replace("add one", "increment"))
    assert bench._code_only("a.hip", code) != bench._code_only("a.hip", code.replace("x + 1", "x + 2"))
    py = "# flags\nFLAGS = ['-O3']  \n"
    assert bench._code_only("b.py", py) == bench._code_only("b.py", "# other words\nFLAGS = ['-O3']\n")
    assert bench._code_only("b.py", py) != bench._code_only("b.py", "FLAGS = ['-O2']\n")


def test_decode_kernel_names():
    # mirrors the library's rule: streamed from 256 MiB of fp32 state, then 4, 2 or 1 column slices
    assert bench.decode_kernel_name(1, 32) == "kda_decode_split4_kernel"
    assert bench.decode_kernel_name(4, 32) == "kda_decode_split4_kernel"
    assert bench.decode_kernel_name(16, 32) == "kda_decode_split2_kernel"
    assert bench.decode_kernel_name(32, 32) == "kda_decode_kernel"
    assert bench.decode_kernel_name(128, 32) == "kda_decode_stream_kernel"
