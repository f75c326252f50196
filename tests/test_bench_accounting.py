"""Algorithmic work that bench.py divides by (CPU).

The per-step byte and flop counts behind every roofline fraction, pinned to
the figures derived independently from the workload shapes in the
measurement plan: phase D (draft pass) and phase S (append 16 + draft) of
the 5-layer Qwen3-8B-shaped drafter.  Bytes count every weight once in bf16
and the injected K/V as fp32; flops count 2 per multiply-add over B rows
per layer, B - 1 rows in the LM head and 4 n_q d B (c + B) in attention.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_diffusion_drafting_pass_amd import inputs as I  # noqa: E402


@pytest.mark.parametrize("name,gbytes,gflops", [
    ("q8b_ctx1024", 3.216, 50.9),      # phase D, context 1024
    ("q8b_ctx8192", 3.510, 60.3),      # phase D, context 8192
])
def test_draft_pass_work(name, gbytes, gflops):
    by, fl = bench.pass_work(I.spec(name))
    assert abs(by / 1e9 - gbytes) < 0.0015
    assert abs(fl / 1e9 - gflops) < 0.05


def test_draft_pass_flops_32_sequences():
    _, fl = bench.pass_work(I.spec("q8b_conc32"))
    assert abs(fl / 1e9 - 1671.8) < 0.1


def test_step_work_context_1024():
    # phase S: the draft pass plus the fusion of 16 appended positions
    # (W_fc once, their features) and their K/V flops
    by, fl = bench.step_work(I.spec("q8b_ctx1024"))
    assert abs(by / 1e9 - 3.385) < 0.0015
    assert abs(fl / 1e9 - 54.9) < 0.05


def test_step_minus_pass_is_the_fusion():
    s = I.spec("q8b_ctx1024")
    by_s, _ = bench.step_work(s)
    by_d, _ = bench.pass_work(s)
    # W_fc (hidden x 5 hidden, bf16) plus 16 rows of bf16 features
    assert by_s - by_d == s.hidden * s.fused_width * 2 + s.block * s.fused_width * 2


def test_lm_head_bytes():
    by, fl = bench.stage_work(I.spec("q8b_ctx1024"), "lm_head", 15)
    assert by == 151936 * 4096 * 2
    assert fl == 2 * 15 * 4096 * 151936


@pytest.mark.parametrize("name,rows,bound", [
    ("q8b_ctx1024", 16, "hbm"),          # 16 rows: 64 flop per weight byte executed
    ("q8b_l3_b32_ragged", 256, "mfma"),  # 8 blocks of 32: 512 flop/B, above the ridge
    ("q8b_conc32", 512, "mfma"),
])
def test_lm_head_executed_intensity(name, rows, bound):
    # executed bf16 flops of one LM-head launch: every padded row, two bf16
    # products per multiply-add (hi/lo activations); the ridge of 2.5 PFLOP/s
    # over 8 TB/s is about 315 flop/B
    s = I.spec(name)
    ef = bench.lm_head_executed_flops(s, s.n_seqs)
    assert ef == 4 * rows * s.vocab * s.hidden
    weight_bytes = s.vocab * s.hidden * 2
    ridge = bench.MFMA_BF16_PEAK_TFS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert ("mfma" if ef / weight_bytes >= ridge else "hbm") == bound
