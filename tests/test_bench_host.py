"""Host checks of bench.py's bookkeeping (no GPU): how a step's kernel trace
is split into stages, including the few-row launches that fold one stage's
work into another, and the per-stage work the roofline divides by."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _k(name, tmpl):
    return f"void ll::(anonymous namespace)::{name}<{tmpl}>(unsigned short const*, int)"


def test_one_block_step_splits_into_the_lattice_stages():
    # the one-block sequence: chunked top-K, node build with the row merge,
    # split-K linears, skinny linears, attention fused with the O projection
    seq = [_k("topk_partial_kernel", "1, 4"), _k("node_build_kernel", "1, 1, false, false, true"),
           _k("gemm_part_kernel", "64, 64, 128"), _k("splitk_resid_rmsnorm_kernel", "8, 1, true")]
    for _ in range(2):
        seq += [_k("gemm_skinny2_kernel", "1"), _k("attention_res_kernel", "128, 128, 4, 4, true"),
                _k("splitk_resid_rmsnorm_kernel", "8, 1, false"), _k("gemm_skinny2_kernel", "2"),
                _k("gemm_part_kernel", "64, 64, 256"), _k("splitk_resid_rmsnorm_kernel", "16, 1, false")]
    seq += [_k("gemm_part_kernel", "64, 64, 64"), _k("splitk_heads_l2norm_kernel", "16, 1"),
            _k("scores_walk_kernel", "0")]
    st = bench.split_step_stages(seq)
    assert st[:4] == ["topk_lse", "node_build", "linear_conf_w2", "linear_conf_w2"]
    layer = ["linear_qkv", "lattice_attention", "linear_o", "linear_ffn1", "linear_ffn2", "linear_ffn2"]
    for l in range(2):
        assert st[4 + 6 * l:10 + 6 * l] == [f"{n}.l{l}" for n in layer]
    assert st[-3:] == ["linear_heads", "linear_heads", "scores_walk"]
    # every linear of the lattice head is found once (the fused attention counts as the O product)
    mains = sum(any(k in n for k in bench._GEMM_MAIN) or bench._fused_attention_o(n) for n in seq)
    assert mains == len(bench._LINEAR_ORDER)


def test_many_row_step_splits_into_the_lattice_stages():
    seq = [_k("topk_partial_kernel", "1, 4"), _k("node_build_kernel", "1, 8, false, false"),
           _k("gemm_dma_kernel", "256, 256, 4, 8"), _k("rmsnorm_reg_kernel", "4")]
    for _ in range(2):
        seq += [_k("gemm_dma_kernel", "256, 256, 1, 8"), _k("attention_res_kernel", "256, 128, 8, 16, false"),
                _k("gemm_dma_kernel", "256, 256, 3, 8"), _k("rmsnorm_reg_kernel", "4"),
                _k("gemm_dma_kernel", "256, 256, 2, 8"), _k("gemm_dma_kernel", "256, 256, 3, 8"),
                _k("rmsnorm_reg_kernel", "4")]
    seq += [_k("gemm_dma_kernel", "256, 256, 0, 8"), _k("splitk_heads_l2norm_kernel", "1, 1"),
            _k("scores_walk_kernel", "0")]
    st = bench.split_step_stages(seq)
    assert st.count("lattice_attention.l0") == 1 and st.count("linear_o.l1") == 2
    assert not bench._fused_attention_o(seq[5])


def test_stage_work_moves_the_o_product_into_the_fused_attention():
    # the one-block workload: the attention stage carries the O product's flops
    # and the O stage is the reduce; summed over both they match the unfused split
    w = synth.WORKLOADS["c1_qwen3_8b"]
    M, H = w.num_blocks * w.slots * w.topk, w.hidden
    att, o = bench.stage_work(w, 4), bench.stage_work(w, 5)
    assert o["flops"] == 0
    T = w.slots * w.topk
    assert att["flops"] == 4 * w.num_blocks * w.heads * T * T * (H // w.heads) + 2 * M * H * H
    # many rows: no fusion, the O stage is the linear
    w3 = synth.WORKLOADS["c256_k16"]
    M3 = w3.num_blocks * w3.slots * w3.topk
    assert bench.stage_work(w3, 5)["flops"] == 2 * M3 * w3.hidden * w3.hidden
