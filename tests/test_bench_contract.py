"""The benchmark's command-line contract, on the CPU (no GPU work)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_sq_summary_derivation(tmp_path):
    """bench.sq_from on a synthetic counter file: the derived figures follow
    from the counters by the stated formulas (T = GRBM_GUI_ACTIVE / 8 XCDs,
    1024 SIMDs, 256 CUs, 4 cycles per VALU issue, per 64 unmasked pairs of the
    d=128 N=8192 causal workload: 2*16*8192^2/2/64 = 16 777 216 groups)."""
    import csv
    import json
    sys.path.insert(0, ROOT)
    import bench
    T = 1_000_000.0
    counters = {"GRBM_GUI_ACTIVE": 8 * T, "SQ_INSTS_VALU": 0.5 * 1024 * T / 4 + 16_777_216.0,
                "SQ_INSTS_MFMA": 16_777_216.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1024 * T,
                "SQ_VALU_MFMA_COEXEC_CYCLES": 0.1 * 1024 * T, "SQ_LDS_IDX_ACTIVE": 0.3 * 256 * T,
                "SQ_WAIT_INST_ANY": 0.2 * 2.5 * 1024 * T / 4, "SQ_ACTIVE_INST_ANY": 0.3 * 2.5 * 1024 * T / 4,
                "SQ_WAVE_CYCLES": 2.5 * 1024 * T / 4,
                "SQ_INSTS_VALU_TRANS_F32": 2 * 16_777_216.0, "SQ_INSTS_SALU": 3 * 16_777_216.0}
    d = tmp_path / "sq"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, k in enumerate(bench.SQ_KERNELS):
            for c, v in counters.items():
                # two rows per counter (e.g. two passes' shares) sum to the value
                w.writerow([i, f"void sage::(anonymous namespace)::{k}<true>(int)", c, v / 2])
                w.writerow([i, f"void sage::(anonymous namespace)::{k}<true>(int)", c, v / 2])
    out = tmp_path / "sq.json"
    doc = bench.sq_from(str(d), out_path=str(out))
    assert json.load(open(out)) == json.loads(json.dumps(doc))
    for k in bench.SQ_KERNELS:
        r = doc["kernels"][k]
        assert abs(r["cycles"] - T) < 1e-6
        assert abs(r["valu_issue_busy"] - (0.5 + 4 * 16_777_216.0 / (1024 * T))) < 1e-9
        assert abs(r["mfma_busy"] - 0.25) < 1e-12 and abs(r["mfma_valu_coexec"] - 0.1) < 1e-12
        assert abs(r["lds_busy"] - 0.3) < 1e-12
        assert abs(r["waves_waiting_on_dependency"] - 0.2) < 1e-12 and abs(r["waves_issuing"] - 0.3) < 1e-12
        assert abs(r["valu_per_64_pairs"] - 0.5 * 1024 * T / 4 / 16_777_216.0) < 1e-9
        assert r["mfma_per_64_pairs"] == 1.0 and r["exp_per_64_pairs"] == 2.0 and r["salu_per_64_pairs"] == 3.0
        assert abs(r["resident_waves_per_simd"] - 2.5) < 1e-12
        assert "valu_classes_per_64_pairs" not in r     # no class counters in this run


def test_sq_summary_valu_classes_and_other_workload(tmp_path):
    """With the per-class VALU counters present, each class is reported per 64
    unmasked pairs and "other" is the VALU count less MFMA and the classes; the
    pair count follows the named workload (d=64 N=2048 causal, B=4, H=16:
    4*16*2048^2/2/64 = 2 097 152 groups) and the file goes beside the
    headline one."""
    import csv
    sys.path.insert(0, ROOT)
    import bench
    g = 2_097_152.0
    T = 1000.0
    counters = {"GRBM_GUI_ACTIVE": 8 * T, "SQ_INSTS_VALU": 12 * g, "SQ_INSTS_MFMA": 1 * g,
                "SQ_VALU_MFMA_BUSY_CYCLES": 1.0, "SQ_VALU_MFMA_COEXEC_CYCLES": 1.0, "SQ_LDS_IDX_ACTIVE": 1.0,
                "SQ_WAIT_INST_ANY": 1.0, "SQ_ACTIVE_INST_ANY": 1.0, "SQ_WAVE_CYCLES": 1.0,
                "SQ_INSTS_SALU": 1.0}
    classes = dict(zip(bench.SQ_VALU_CLASSES, (1.0, 0.5, 3.0, 1.0, 2.0, 2.5, 0.0)))
    for c, x in classes.items():
        counters[c] = x * g
    d = tmp_path / "sq"
    d.mkdir()
    with open(d / "y_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, k in enumerate(bench.SQ_KERNELS):
            for c, v in counters.items():
                w.writerow([i, f"void sage::(anonymous namespace)::{k}<false>(int)", c, v])
    assert bench.sq_file("d64_n2k_causal").endswith("profiles/sq_utilisation_d64_n2k_causal.json")
    assert bench.sq_file(bench.HEADLINE_WORKLOAD) == bench.SQ_FILE
    doc = bench.sq_from(str(d), "d64_n2k_causal", out_path=str(tmp_path / "o.json"))
    assert doc["workload"] == "d64_n2k_causal"
    for k in bench.SQ_KERNELS:
        r = doc["kernels"][k]
        assert abs(r["valu_per_64_pairs"] - 11.0) < 1e-12 and abs(r["mfma_per_64_pairs"] - 1.0) < 1e-12
        cls = r["valu_classes_per_64_pairs"]
        assert abs(cls["FMA_F32"] - 3.0) < 1e-12 and abs(cls["INT32"] - 2.5) < 1e-12
        assert abs(cls["other"] - (11.0 - 10.0)) < 1e-12


def test_backward_roofline_prices_each_product_at_its_own_peak():
    """d=128 N=8192 causal (B=2, H=16): 2^30 unmasked pairs, 8*128 INT8
    operations and 2*128 BF16 flops per pair; at 5.0 POP/s and 2.5 PFLOP/s
    the ideal time is 219.9 + 110.0 us, so the mixed ceiling is
    5*2^38 ops / 329.9 us = 4166.7 TOP/s."""
    sys.path.insert(0, ROOT)
    import bench
    from bit_trainable_attention_block_amd import workloads as wl
    w = bench.bwd_work(wl.C3)
    pairs = 2 * 16 * 8192 * 8192 / 2
    assert w == {"int8_ops": 8 * 128 * pairs, "bf16_flops": 2 * 128 * pairs}
    assert abs(bench.mixed_ceiling_tops(w) - 5 / (4 / 5000 + 1 / 2500)) < 1e-9
    assert abs(bench.mixed_ceiling_tops(w) - 4166.67) < 0.01
    assert bench.bwd_pre_algo_bytes(128) == 5.03125 and bench.QUANT_ALGO_BYTES == 11.0


def test_cpu_sweep_head_sample_is_spread_and_valid():
    """The CPU sweep's head sample: distinct (batch, head) pairs inside the
    workload, evenly spread, all heads when there are fewer than asked."""
    sys.path.insert(0, ROOT)
    import bench
    from bit_trainable_attention_block_amd import workloads as wl
    for cfg in (wl.C1, wl.C2, wl.C3, wl.C4[0], wl.C5):
        hs = bench.sample_heads(cfg, 16)
        assert len(hs) == min(16, cfg.B * cfg.H) == len(set(hs))
        assert all(0 <= b < cfg.B and 0 <= h < cfg.H for b, h in hs)
    assert bench.sample_heads(wl.C2, 16)[:5] == [(0, 0), (0, 4), (0, 8), (0, 12), (1, 0)]   # 64 heads, step 4
    assert bench.sample_heads(wl.C5, 16) == [(0, h) for h in range(8)]                        # all 8
