"""Host-side pieces of bench.py (CPU only): the source stamp that decides
whether committed HBM-traffic counters still describe the built kernels."""
import bench


def test_code_only_drops_comments_and_layout_keeps_literals():
    a = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x /*y*/"; char c = \'"\';'
    b = 'int a = 1;\n\n   const char* s = "//x /*y*/";   char c = \'"\'; // other note'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) == 'int a = 1; const char* s = "//x /*y*/"; char c = \'"\';'
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 64


def test_attention_flops_counts_visible_pairs():
    import numpy as np
    import workloads
    cfg = workloads.config("prefix_verify", batch=2, q_len=3)
    lens = np.array([10, 20])
    per_pair = 4 * cfg.num_q_heads * cfg.head_dim
    # a chain: row i sees L - q_len + i + 1 tokens
    assert bench.attention_flops(cfg, lens) == per_pair * sum(L - 3 + i + 1 for L in (10, 20) for i in range(3))
    # every drafted token hangs off the context: each sees the context and itself
    flat = np.full((2, 3), -1)
    assert bench.attention_flops(cfg, lens, flat) == per_pair * 3 * ((10 - 2) + (20 - 2))
    # a chain written as parents equals the causal count
    chain = np.array([[-1, 0, 1], [-1, 0, 1]])
    assert bench.attention_flops(cfg, lens, chain) == bench.attention_flops(cfg, lens)


def test_counter_summary_means_rates_and_stamp(tmp_path):
    """Per-launch means of the main kernel's counters from rocprofv3 CSVs
    (other kernels ignored), the MFMA rate at the bench line's launch time,
    and the stamp that ties the summary to the current sources."""
    import csv
    import json
    kernel = "mfma_attn_balanced<128, 16, 2, false, false, false>"
    rows = [("void (anonymous namespace)::" + kernel + "((anonymous namespace)::AttnArgs)", "MfmaFlopsBF16", v)
            for v in (4.0e10, 4.2e10)]
    rows += [("void (anonymous namespace)::" + kernel + "((anonymous namespace)::AttnArgs)", "MfmaUtil", v)
             for v in (7.0, 7.2)]
    rows += [("at::native::fill_kernel", "MfmaUtil", 99.0)]
    run = tmp_path / "run_mfma"
    run.mkdir()
    with open(run / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writerows(rows)
    line = {"roofline": {"kernel": kernel, "launch_us": 200.0}, "flops": 2.5e10}
    (tmp_path / "bench.json").write_text(json.dumps(line) + "\n")
    out = bench.counter_summary("wl", [str(run)], str(tmp_path / "bench.json"), out_dir=str(tmp_path))
    assert out["per_launch"]["MfmaUtil"] == 7.1 and out["dispatches"]["MfmaUtil"] == 2
    assert abs(out["mfma_bf16_tflops"] - 4.1e10 / 200e-6 / 1e12) < 1e-9
    assert abs(out["mfma_bf16_frac_of_peak"] - out["mfma_bf16_tflops"] / 2500.0) < 1e-12
    assert abs(out["mfma_flops_over_algorithmic"] - 4.1e10 / 2.5e10) < 1e-12
    got = bench.committed_counters("wl", kernel, profiles_dir=str(tmp_path))
    assert got["mfma_util_pct"] == 7.1 and got["source"] == "profiles/counters_wl.json"
    assert bench.committed_counters("wl", "another_kernel<1>", profiles_dir=str(tmp_path)) is None
    stale = json.loads((tmp_path / "counters_wl.json").read_text())
    stale["source_sha256"] = "0" * 64
    (tmp_path / "counters_wl.json").write_text(json.dumps(stale))
    assert bench.committed_counters("wl", kernel, profiles_dir=str(tmp_path)) is None
