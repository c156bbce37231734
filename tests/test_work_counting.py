"""The flop convention used for every throughput figure, pinned to the pages'
per-tile cycle table (tests/golden/pages_constants.json), and the seeded input
recipe."""
import json
import math
import os

import torch

import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def test_cycle_model_reproduces_printed_table():
    t = GOLD["tile"]
    feeds = GOLD["feeds_b200"]
    c = workloads.tile_cycles(t["m"], t["n"], t["d"], feeds["mma_ops_per_clk"],
                              feeds["exp_ops_per_clk"])
    assert c["mma_fwd"] == GOLD["fwd_cycles"]["mma"]
    assert c["exp"] == GOLD["fwd_cycles"]["exp"] == GOLD["bwd_cycles_1cta"]["exp"]
    assert c["mma_bwd"] == GOLD["bwd_cycles_1cta"]["mma"]
    assert c["mma_bwd"] / c["mma_fwd"] == GOLD["bwd_over_fwd_mma"]["value"]


def test_flops_convention():
    f = workloads.attention_flops([4096] * 4, [4096] * 4, 16, 128, causal=False)
    assert f["fwd"] == 4 * 4 * 16 * 4096 * 4096 * 128
    assert f["bwd"] == 2.5 * f["fwd"]
    fc = workloads.attention_flops([8192] * 2, [8192] * 2, 16, 128, causal=True)
    assert fc["fwd"] == 0.5 * 4 * 2 * 16 * 8192 * 8192 * 128
    w = workloads.WORKLOADS["causal8k"]
    assert workloads.workload_flops(w) == fc


def test_tau_is_log2_256():
    assert GOLD["tau"]["value"] == math.log2(256)


def test_inputs_are_seeded_bf16_and_scaled():
    a = workloads.make_inputs(1, 16, 16, 4, 4, 8, seed=3, scaled_heads=True)
    b = workloads.make_inputs(1, 16, 16, 4, 4, 8, seed=3, scaled_heads=True)
    for n in ("q", "k", "v", "do"):
        assert a[n].dtype == torch.bfloat16
        assert torch.equal(a[n], b[n])
    assert a["q"][..., :2, :].float().std() > 2.0 * a["q"][..., 2:, :].float().std()


def test_varlen_lengths_in_range():
    w = workloads.WORKLOADS["varlen_gqa"]
    lens = workloads.draw_lengths(w.num_seqs, w.len_lo, w.len_hi, 71004)
    assert len(lens) == 16 and min(lens) >= 512 and max(lens) <= 8192
    cu = workloads.cu_from_lengths(lens)
    assert cu.dtype == torch.int32 and cu[-1].item() == sum(lens)
