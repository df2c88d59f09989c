"""The benchmark's accounting (CPU only): the algorithmic flops and bytes behind its roofline entry
and its throughput figures, recomputed by hand from the workload shapes and the method's
per-element work, and its refusal of more than one GPU."""
import subprocess
import sys

import pytest

import bench
from block_scale_search_amd import workloads

C = workloads.CONFIGS


def test_window_search_work_on_the_70b_matrices():
    # WMSE [-9,6]: 16 codes x 16 elements per group; per element and code the method does
    # x = |w| r (1 flop), the residual fma (2), the weighting multiply (1) and the accumulating
    # fma (2): 6 flops; as VALU lane-operations (rounding included, fma = 1): 5
    for name in ("mlp70b_up", "mlp70b_down"):
        cfg = C[name]
        n_w = 28672 * 8192
        assert cfg.n_weights == n_w
        flops, ops = bench.search_work(cfg, f"{name}/search:WMSE [-9,6]")
        assert flops == n_w * 16 * 6 == 22_548_578_304
        assert ops == n_w * 16 * 5
        # read W (bf16) and h once, write 4-bit codes and one scale byte per 16 weights
        assert bench.algorithmic_bytes(cfg, "search:WMSE [-9,6]") == \
            n_w * 2 + n_w // 2 + n_w // 16 + cfg.inp * 4


def test_exhaustive_counts_the_codes_it_scores():
    # the pruned search's work is the (group, code) candidates it scores, 16 elements each
    cfg = C["mlp70b_up"]
    scored = 40 * (cfg.n_weights // 16)
    flops, ops = bench.search_work(cfg, "search:WMSE exhaustive(126)", scored)
    assert flops == scored * 16 * 6
    assert ops == scored * 16 * 5
    assert bench.centre_lo(cfg, "search:WMSE exhaustive(126)") == -8


def test_fused_window_and_exhaustive():
    # the 70B matrices' two modes are one launch; the window is the exhaustive search's first
    # block, so the launch's work is the exhaustive search's alone, and both outputs are written
    for name in ("mlp70b_up", "mlp70b_down", "tiny"):
        cfg = C[name]
        pair = bench.paired_modes(cfg)
        assert [m.label for m in pair] == ["WMSE [-9,6]", "WMSE exhaustive(126)"]
        label = bench.pair_label(pair)
        assert bench.centre_lo(cfg, label) == -9
        assert "k_scale_search_exhaustive" in bench.kernel_name(cfg, label)
        n_w = cfg.n_weights
        scored = 33 * (n_w // 16)
        flops, _ = bench.search_work(cfg, label, scored)
        assert flops == scored * 16 * 6
        wb = 2 if bench.is_bf16(cfg) else 4
        assert bench.algorithmic_bytes(cfg, label) == \
            n_w * wb + 2 * (n_w // 2 + n_w // 16) + cfg.batch * cfg.inp * 4


def test_paired_launch_counts_both_rules():
    cfg = C["attn8b"]
    assert [m.label for m in bench.paired_modes(cfg)] == ["MSE [-3,7]", "WMSE [-8,7]"]
    label = bench.pair_label(bench.paired_modes(cfg))
    # MSE [-3,7] lies inside WMSE [-8,7]: one scan of the 16 codes serves both
    assert bench.kernel_name(cfg, label).startswith("k_scale_search_nested")
    flops, ops = bench.search_work(cfg, label)
    n_w = 4096 * 4096
    assert flops == n_w * (11 * 5 + 16 * 6)
    assert ops == n_w * (11 * 4 + 16 * 5)
    # W and h read once for both rules, each rule's codes and scales written
    assert bench.algorithmic_bytes(cfg, label) == n_w * 2 + 2 * (n_w // 2 + n_w // 16) + 4096 * 4


def test_h_stage_bytes():
    up, down = C["mlp70b_up"], C["mlp70b_down"]
    # all resident chunks in one call: X once, plus h_acc in/out and h per column
    assert bench.algorithmic_bytes(up, "h_reduce_chunks") == 65536 * 8192 * 2 + 8192 * 12
    assert bench.algorithmic_bytes(down, "h_reduce_chunks") == 65536 * 28672 * 2 + 28672 * 12
    # one deferred chunk call reads its chunk only
    assert bench.algorithmic_bytes(up, "h_reduce") == 8192 * 8192 * 2
    # h and S of a one-chunk layer in one call: X, W and the per-column outputs
    attn = C["attn8b"]
    assert bench.algorithmic_bytes(attn, "h_reduce+global_scale") == \
        8192 * 4096 * 2 + 4096 * 12 + 4096 * 4096 * 2 + 4


def test_the_pair_workload_is_both_70b_matrices():
    cfgs = workloads.workload_configs("mlp70b")
    assert [c.name for c in cfgs] == ["mlp70b_up", "mlp70b_down"]
    assert all([m.label for m in c.modes] == ["WMSE [-9,6]", "WMSE exhaustive(126)"] for c in cfgs)
    assert all(c.chunk_tokens == 8192 and c.tokens == 65536 for c in cfgs)
    assert bench.DEFAULT_WORKLOAD == "mlp70b"


def test_peaks():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-operations; x2 for an fma, x2 for packed fp32
    assert abs(256 * 4 * 16 * 2.4e9 / 1e12 - bench.VALU_ISSUE_TOPS) < 0.01
    assert abs(bench.VALU_ISSUE_TOPS * 4 - bench.VALU_PUBLISHED_TFLOPS) < 0.05
    assert bench.HBM_PEAK_GBS == 8000.0


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", n], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
