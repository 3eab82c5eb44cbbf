"""Host-side pieces of bench.py: the algorithmic byte counts and the
rocprofv3 counter summary (no GPU)."""
import csv
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_attention_bytes_counts_kv_q_out_and_table():
    # one sequence of 17 tokens, 1 kv head, 2 q heads: K and V of 17 tokens
    # (64 BF16 values each), q BF16 in, FP32 out, two block-table entries
    got = bench.attention_bytes([17], Hq=2, Hkv=1, q_bytes=2)
    assert got == 17 * 64 * 2 * 2 + 2 * 64 * (2 + 4) + 2 * 4


def test_step_bytes_is_weights_plus_attention_plus_io():
    shape = synth.tiny_shape(hidden=128, layers=2, heads=4, kv_heads=2, inter=256, vocab=1000)
    lens = np.array([5, 40])
    per_layer = (2 * shape.layer_param_count() + bench.attention_bytes(lens, 4, 2, 4)
                 + 2 * 2 * 64 * 2 * 2 + 2 * 2 * 128 * 4)
    want = 2 * per_layer + 2 * 128 * 2 + 2 * 1000 * 128 + 128 * 2 + 2 * 1000 * 4
    assert bench.step_bytes(shape, lens) == want


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v])


def test_traffic_summary_scales_by_the_copy(tmp_path):
    mib = bench.COPY_BYTES / 2.0 ** 20
    att = "void pkv::(anonymous namespace)::paged_attention_kernel<unsigned short>(pkv::AttnArgs)"
    mrg = "pkv::(anonymous namespace)::attention_merge_kernel(pkv::AttnArgs)"
    # small copies, then the calibration copy, which the counter reads as
    # 1.25x its size; attention reads 1000 and
    # 1200 KiB (mean 1100), the merge 100 KiB
    _write_counters(tmp_path / "f.csv", [
        ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 3.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 4.0),
        ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.25 * mib * 1024),
        (att, "FETCH_SIZE", 1000.0), (att, "FETCH_SIZE", 1200.0), (mrg, "FETCH_SIZE", 100.0)])
    _write_counters(tmp_path / "w.csv", [
        ("__amd_rocclr_copyBuffer", "WRITE_SIZE", mib * 1024),
        (att, "WRITE_SIZE", 40.0), (mrg, "WRITE_SIZE", 8.0)])
    out = tmp_path / "t.json"
    bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out_path=str(out))
    t = json.load(open(out))
    assert abs(t["fetch_scale"] - 0.8) < 1e-9
    assert t["fetch_bytes_per_launch"] == round((1100.0 + 100.0) * 1024 * 0.8)
    assert t["write_bytes_per_launch"] == round(48.0 * 1024)
    assert t["attention_source_sha"] == bench.source_sha(bench.ATTN_SOURCE)


def test_counter_table_scales_each_library_kernel(tmp_path, capsys):
    mib = bench.COPY_BYTES / 2.0 ** 20
    gate = "void pkv::(anonymous namespace)::gemm_kernel<1, 2, 4, 2, false>(pkv::GemmArgs)"
    red = "pkv::(anonymous namespace)::resid_reduce_kernel(float const*, int, int, int, float const*, float*, float*)"
    # the copy reads as half its size (scale 2) for FETCH, its size for WRITE;
    # torch's own kernels are left out
    _write_counters(tmp_path / "f.csv", [
        ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 0.5 * mib * 1024),
        (gate, "FETCH_SIZE", 1000.0), (gate, "FETCH_SIZE", 3000.0), (red, "FETCH_SIZE", 10.0),
        ("at::native::vectorized_elementwise_kernel", "FETCH_SIZE", 5.0)])
    _write_counters(tmp_path / "w.csv", [
        ("__amd_rocclr_copyBuffer", "WRITE_SIZE", mib * 1024),
        (gate, "WRITE_SIZE", 100.0), (gate, "WRITE_SIZE", 100.0), (red, "WRITE_SIZE", 20.0)])
    bench.counter_table(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    lines = capsys.readouterr().out.strip().splitlines()
    rows = {ln.split("|")[1].strip(): ln for ln in lines[2:]}
    assert set(rows) == {"gemm_kernel<1, 2, 4, 2, false>", "resid_reduce_kernel"}
    g = [c.strip() for c in rows["gemm_kernel<1, 2, 4, 2, false>"].split("|")[2:5]]
    assert g == ["2", "%.3f" % (2000.0 * 1024 * 2 / 1e6), "%.3f" % (100.0 * 1024 / 1e6)]
    assert lines[2].startswith("| gemm_kernel")  # largest fetch first


def test_prefill_flops_counts_projections_causal_attention_and_one_head_row():
    s = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    start, T = 5, 3
    H, D = s.hidden, s.head_dim
    per_token = 2 * ((s.heads + 2 * s.kv_heads) * D * H + s.heads * D * H + 3 * s.inter * H)
    keys = (start + 1) + (start + 2) + (start + 3)
    per_layer = T * per_token + 4 * s.heads * D * keys
    assert bench.prefill_flops(s, start, T) == s.layers * per_layer + 2 * s.vocab * H
