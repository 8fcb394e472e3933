"""Host-side checks of bench.py's contract (no GPU needed).

The algorithmic byte and FLOP counts are the fixed per-unit figures of the
measurement plan: 1796 B per token-head for prefill (q, k, v bf16, log_g and
out fp32, beta), plus the initial and final state once per unit; two state
passes per unit plus 1796 B per row for kda_step; 5*2*C*d + 3*2*d*d FLOP per
token-head for the chunked form.
"""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_bytes_and_flops_of_the_dense_workload():
    tokens, H, d = 4 * 4096, 16, 128
    # 16384 tokens x 16 heads x 1796 B + 2 x 4 sequences x 16 heads x 64 KiB
    assert bench.prefill_bytes(tokens, H, d, n_states=4) == 16384 * 16 * 1796 + 2 * 4 * 16 * 65536
    assert bench.prefill_bytes(tokens, H, d, n_states=4) == 479_199_232
    assert bench.prefill_flops(tokens, H, d) == 16384 * 16 * 180_224 == 47_244_640_256


def test_step_bytes_of_decode_and_verify():
    # 2 x 64 KiB of state per unit plus one 1796-byte row per token-head
    assert bench.step_bytes(256, 1, 32, 128) == 256 * 32 * (2 * 65536 + 1796) == 1_088_454_656
    assert bench.step_bytes(64, 4, 32, 128) == 64 * 32 * (2 * 65536 + 4 * 1796) == 283_148_288


def test_rows_and_commit_bytes_of_the_verify_workload():
    # rows: the state read once, each row's q, k, v (bf16), log_g, beta, out and delta
    per_row = 3 * 256 + 512 + 4 + 512 + 512
    assert bench.rows_bytes(64, 4, 32, 128) == 64 * 32 * (65536 + 4 * per_row) == 153_124_864
    # commit: the state read and written, each row's k (bf16), log_g and delta, the accept counts
    assert bench.commit_bytes(64, 4, 32, 128) == 64 * 32 * (2 * 65536 + 4 * (256 + 512 + 512)) + 64 * 4
    assert bench.commit_bytes(64, 4, 32, 128) == 278_921_472


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def _write_counter_csv(dirname, counter, rows, grid=1024):
    """rows: (kernel name, dispatch id, value) or (..., grid size in threads)."""
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Dispatch_Id", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for row in rows:
            name, disp, val = row[:3]
            w.writerow({"Kernel_Name": name, "Dispatch_Id": disp, "Grid_Size": row[3] if len(row) > 3 else grid,
                        "Counter_Name": counter, "Counter_Value": val})


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    # the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    _write_counter_csv(tmp_path / "cf", "FETCH_SIZE", [("copy_kernel", 1, kib / 2), ("tiny", 2, 1.0)])
    _write_counter_csv(tmp_path / "cw", "WRITE_SIZE", [("copy_kernel", 1, kib)])
    # two dispatches of each prefill kernel: the mean per dispatch is used
    _write_counter_csv(tmp_path / "pf", "FETCH_SIZE", [("prep_kernel(x)", 1, 100.0), ("prep_kernel(x)", 3, 300.0),
                                                       ("scan_kernel(y)", 2, 50.0), ("scan_kernel(y)", 4, 50.0)])
    _write_counter_csv(tmp_path / "pw", "WRITE_SIZE", [("prep_kernel(x)", 1, 10.0), ("prep_kernel(x)", 3, 10.0),
                                                       ("scan_kernel(y)", 2, 20.0), ("scan_kernel(y)", 4, 20.0)])
    lines = bench.write_traffic(str(tmp_path / "pf"), str(tmp_path / "pw"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    kv = dict(l.split(": ", 1) for l in lines)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0, rel=1e-4)
    assert float(kv["write_scale"]) == pytest.approx(1.0, rel=1e-4)
    prep = (200.0 * 2.0 + 10.0) * 1024
    scan = (50.0 * 2.0 + 20.0) * 1024
    assert int(kv["prep_kernel_bytes"]) == round(prep)
    assert int(kv["scan_kernel_bytes"]) == round(scan)
    assert int(kv["traffic_bytes_per_call"]) == round(prep + scan)
    assert kv["sources_sha256"] == bench.sources_hash()


@pytest.mark.parametrize("kind", ["prefill", "backward"])
def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch, kind):
    f = tmp_path / "traffic.txt"
    monkeypatch.setitem(bench.TRAFFIC[kind], "file", str(f))
    f.write_text(f"# comment\nsources_sha256: {bench.sources_hash(kind)}\ntraffic_bytes_per_call: 123456\n")
    assert bench.read_traffic(kind) == 123456
    f.write_text("sources_sha256: 0000000000000000\ntraffic_bytes_per_call: 123456\n")
    assert bench.read_traffic(kind) is None
    f.unlink()
    assert bench.read_traffic(kind) is None


def test_source_stamp_ignores_comments_but_not_code():
    """A traffic or MFMA summary stays valid across comment edits of the
    kernel sources and lapses with any change to their code."""
    code = "int f(int x) {  // doubled\n  return 2 * x;\n}\n"
    assert bench.code_only(code) == bench.code_only("/* header\n over two lines */\n" + code.replace("doubled", "x2"))
    assert bench.code_only(code) == bench.code_only(code.replace("\n", "\n\n"))
    assert bench.code_only(code) != bench.code_only(code.replace("2 * x", "3 * x"))
    assert bench.code_only(code) != bench.code_only(code.replace("return", "return -"))


def test_decode_traffic_counts_only_the_decode_dispatches(tmp_path):
    """The decode instantiation also serves verify's one-row reference at a
    quarter of the units: only dispatches of the decode grid are averaged."""
    kib = bench.COPY_BYTES / 1024.0
    _write_counter_csv(tmp_path / "cf", "FETCH_SIZE", [("copy_kernel", 1, kib / 2)])
    _write_counter_csv(tmp_path / "cw", "WRITE_SIZE", [("copy_kernel", 1, kib)])
    dec, ref = "void recurrent_kernel<128, 128, bf16_t, false>(RecArgs)", 256 * 32 * 512
    other = "void recurrent_kernel<128, 64, bf16_t, false>(RecArgs)"
    _write_counter_csv(tmp_path / "sf", "FETCH_SIZE", [(dec, 1, 100.0, ref), (dec, 2, 25.0, ref // 4),
                                                       (dec, 3, 100.0, ref), (other, 4, 7.0, ref // 2)])
    _write_counter_csv(tmp_path / "sw", "WRITE_SIZE", [(dec, 1, 200.0, ref), (dec, 2, 50.0, ref // 4),
                                                       (dec, 3, 200.0, ref)])
    lines = bench.write_traffic(str(tmp_path / "sf"), str(tmp_path / "sw"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                                kind="decode")
    kv = dict(l.split(": ", 1) for l in lines)
    assert int(kv["traffic_bytes_per_call"]) == round((100.0 * 2.0 + 200.0) * 1024)


def test_backward_traffic_sums_the_five_backward_kernels(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    _write_counter_csv(tmp_path / "cf", "FETCH_SIZE", [("copy_kernel", 1, kib)])
    _write_counter_csv(tmp_path / "cw", "WRITE_SIZE", [("copy_kernel", 1, kib)])
    names = ["bwd_prep<128>", "bwd_fscan3<128>", "bwd_rscan3<128>", "bwd_gstate<128>", "bwd_gpairs<128>"]
    _write_counter_csv(tmp_path / "bf", "FETCH_SIZE", [(n, i, 10.0 * (i + 1)) for i, n in enumerate(names)] +
                       [("prep_kernel(x)", 9, 1000.0)])
    _write_counter_csv(tmp_path / "bw", "WRITE_SIZE", [(n, i, 1.0) for i, n in enumerate(names)])
    lines = bench.write_traffic(str(tmp_path / "bf"), str(tmp_path / "bw"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                                kind="backward")
    kv = dict(l.split(": ", 1) for l in lines)
    assert int(kv["traffic_bytes_per_call"]) == round((10 + 20 + 30 + 40 + 50 + 5) * 1024)
    assert kv["sources_sha256"] == bench.sources_hash("backward")
    assert bench.sources_hash("backward") != bench.sources_hash("prefill")


def test_backward_bytes_and_flops_of_the_dense_workload():
    tokens, H, d = 4 * 4096, 16, 128
    # q, k, v bf16, log_g, beta, d_out in; dq, dk, dv, dlog_g fp32 and dbeta out: 3848 B per
    # token-head; init_state and d_final in, d_init_state out per unit
    assert bench.backward_bytes(tokens, H, d, n_states=4) == tokens * H * 3848 + 3 * 4 * 16 * 65536
    # per 64-token chunk: 64^3/6 + 6 * 64^2 * 128 + 8 * 64 * 128^2 multiply-adds
    macs = 64 ** 3 // 6 + 6 * 64 * 64 * 128 + 8 * 64 * 128 * 128
    assert macs == 11_578_026
    assert bench.backward_flops(tokens, H, d) == tokens * H * 2 * macs // 64 == 94_847_188_992


def test_conv_bytes_of_the_qkv_workload():
    # 4 x 4096 tokens x 6144 channels of bf16 read and written, weights, final caches
    assert bench.conv_bytes(4 * 4096, 6144, 4, 4) == 16384 * 6144 * 4 + 6144 * 4 * 4 + 4 * 6144 * 3 * 4


def test_norm_bytes_of_the_output_workload():
    # 262144 rows of 128: fp32 o and bf16 gate read, bf16 out written; the weight
    assert bench.norm_bytes(4 * 4096 * 16, 128) == 262144 * 128 * 8 + 512
