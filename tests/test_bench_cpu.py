"""Host logic of bench.py, on the CPU: the work and byte models the benchmark line
reports against, and its refusal of a multi-GPU run.

The per-head-token figures are those worked out by hand for the three forward
workloads (algorithmic flops of the chunked forward: summaries, scan combines
and chunk outputs at full chunk tiles; minimal bytes: q, k, v read once and
the output written once).
"""
import bench
from causal_prefix_scan_hla2_amd import inputs as I


def test_forward_flop_model_matches_hand_figures():
    # normalised 2k (d = dv = 64, ratio, chunk 64), decay 8k (d = 64, dv = 128, chunk 64),
    # long 64k (d = dv = 128, ratio, chunk 128)
    assert bench.canonical_flops_per_head_token(64, 64, 64, True) == 115712
    assert bench.canonical_flops_per_head_token(64, 128, 64, False) == 180224
    assert bench.canonical_flops_per_head_token(128, 128, 128, True) == 460800


def test_forward_min_bytes():
    w = I.WORKLOADS["decay_8k"]
    # 8 x 16 heads x 8192 tokens x (q, k: 64 + 64; v, out: 128 + 128) bf16 elements
    assert bench.min_bytes_forward(w, 2) == 8 * 16 * 8192 * 384 * 2 == 805306368


def test_output_launch_bytes_under_a_lead_plan():
    w = I.WORKLOADS["decay_8k"]
    plan = (3, 34, 48, True)  # segments, chunks of segment 0, chunks of the others, lead
    tokens = 8192 - 34 * 64
    assert bench.output_launch_tokens(w, plan) == tokens
    state = (64 * 64 + 64 * 128 + 64) * 4  # S0, U0, u0 in fp32, read by segments 1 and 2
    # segment 1's summary S, C, U, m, u in fp32, read once by segment 2's workgroups (their prologue fold)
    summary = (64 * 64 + 2 * 64 * 128 + 2 * 64) * 4
    assert bench.prologue_folds(w, plan) == 1
    assert bench.output_kernel_bytes(w, 2, plan) == \
        8 * 16 * tokens * 384 * 2 + 8 * 16 * 2 * state + 8 * 16 * summary == 614596608
    # a plan with more segments launches the scan: no fold in the output launch
    assert bench.prologue_folds(w, (5, 20, 27, True)) == 0
    # a plain plan walks every token in the output launch
    assert bench.output_launch_tokens(w, (4, 32, 32, False)) == 8192


def test_roofline_picks_the_binding_bound():
    # 1 GB and 1 TFLOP in 1 ms: intensity 1000 flop/B, above the 312.5 flop/B ridge -> MFMA
    r = bench.roofline(1e12, 1e9, 1e-3)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and abs(r["achieved"] - 1000.0) < 1e-9
    # 1 GB and 10 GFLOP: 10 flop/B -> HBM, 1 TB/s achieved = 1/8 of the peak
    r = bench.roofline(1e10, 1e9, 1e-3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["frac"] - 0.125) < 1e-12


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
