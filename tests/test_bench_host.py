"""Host-side logic of bench.py (CPU only): the one-GPU rule, the algorithmic byte and flop counts
that every roofline fraction divides by (checked against counts written out by hand for the
batch-1 workload: 2048-token prefix, S = 16, 32 query / 2 kv heads, head_dim 128, LM head
2688 x 131072, bf16, and for the default batch-4 128K workload), and the LM-head kernel label."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_of_the_batch1_workload():
    a = bench.algorithmic(synth.workload(1))
    kv_rows = 2 * 2048 * 128 * 2 * 2          # 2 kv heads x 2048 rows x 128 dims x 2 B, K and V
    q_and_o = 2 * (16 * 32 * 128 * 2)         # 16 positions x 32 heads x 128 dims x 2 B, Q and O
    block_kv = 16 * 2 * 128 * 2 * 2           # the block's own K and V rows
    assert a["attn_bytes"] == kv_rows + q_and_o + block_kv == 2_375_680
    # scores and PV: 256 query rows (16 positions x 16 grouped heads) per kv head, 2064 keys each
    assert a["attn_flops"] == 2 * (2 * 256 * 128 * 2064) * 2 == 541_065_216
    w_bytes = 131072 * 2688 * 2
    assert a["lm_bytes"] == w_bytes + 16 * 2688 * 2 + 16 * 131072 * 4 == 713_117_696
    assert a["lm_flops"] == 2 * 16 * 2688 * 131072


def test_algorithmic_counts_scale_with_the_prefix_sum():
    """Ragged prefixes enter only through their sum: K/V bytes and flops grow linearly with it."""
    w1 = synth.workload(1, B=3, prefixes=[100, 200, 300])
    w2 = synth.workload(1, B=3, prefixes=[600, 0, 0])
    a1, a2 = bench.algorithmic(w1), bench.algorithmic(w2)
    assert a1["attn_bytes"] == a2["attn_bytes"] and a1["attn_flops"] == a2["attn_flops"]
    w3 = synth.workload(1, B=3, prefixes=[700, 0, 0])
    a3 = bench.algorithmic(w3)
    assert a3["attn_bytes"] - a2["attn_bytes"] == 100 * 2 * 2 * 128 * 2


def test_algorithmic_counts_of_the_default_workload():
    a = bench.algorithmic(synth.workload(4))
    # per layer: 2 kv heads x 4 x 131072 rows x 128 dims x 2 B, K and V; Q, O, block K/V as above x 4
    assert a["attn_bytes"] == 2 * 4 * 131072 * 128 * 2 * 2 + 4 * (2 * 16 * 32 * 128 * 2 + 16 * 2 * 128 * 2 * 2)
    assert a["attn_bytes"] == 537_985_024
    assert a["lm_bytes"] == 131072 * 2688 * 2 + 64 * 2688 * 2 + 64 * 131072 * 4


def test_default_workload_is_the_largest_one_gpu_workload():
    sys_argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        assert bench.parse().workload == 4
    finally:
        sys.argv = sys_argv


def test_lmhead_kernel_label_follows_the_library_choice():
    """The kernel tt_lmhead_logits picks (lmhead.hip lm_use_lds / gemm.hip gemm_cfg), per workload."""
    name = bench.lmhead_kernel_name
    assert name(16, 2688, 131072) == "lmhead_lds_kernel"          # batch 1
    assert name(128, 2688, 131072) == "lmhead_gemm_kernel<1, 4, 4>"     # batch 8
    assert name(512, 2688, 131072) == "lmhead_gemm_kernel<2, 4, 4>"     # ragged batch 32
    assert name(64, 2688, 131072) == "lmhead_gemm_kernel<1, 2, 2>"      # batch 4
    assert name(17, 2688, 131072) == "lmhead_gemm_kernel<1, 2, 2>"
    assert name(64, 2688, 16384) == "lmhead_lds_kernel"           # small vocabulary
    assert name(128, 256, 32768) == "lmhead_gemm_kernel<2, 4, 4>"
    assert name(16, 96, 2000) == "lmhead_kernel"
    assert name(16, 64, 1024, "f32") == "lmhead_kernel"
