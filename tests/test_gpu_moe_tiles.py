"""GPU parity of the grouped tile classes against the oracle.

The grouped projections cut each expert's rows into 256-row tiles, one
remainder tile of 256 rows (remainder > 128) or 128 rows (65-128), and 16-row
weight-streaming tiles (<= 64).  These tests put rows into every class and
check them with the staged protocol (tests/moe_check.py):

* a small layer whose Zipf-skewed routing gives 54-914 rows per expert, every
  row checked, with general (quantized) and power-of-two (MXFP4-remapped)
  weight scales;
* the 384-expert prefill (T = 16384, H = 7168, I = 2048, experts remapped from
  MXFP4) at full size, on rows stratified by tile class (page
  "DeepSeek-V4.1-Flash-NVFP4", sections 一 and 三: 384 routed experts w1/w3/w2
  from MXFP4; page "Qwen3.8-Flash-Next-NVFP4", section 核心: W4A4);
* the 384-expert decode batch (T = 64) on every row;
* the 512-expert top-10 layer (T = 4096) on stratified rows;
* the 27B-class MLP (hidden 5120, intermediate 17408; page
  "Qwen3.8-27B-NVFP4", section 2) at M = 8192 as a one-expert layer.
"""
import numpy as np
import pytest

from precision_moe_gemm_amd import synth
from tests.gpu_util import step
from tests.moe_check import check_moe_rows, tile_class_rows

pytestmark = pytest.mark.gpu

SKEWED = synth.MoE(seed=50, E=8, k=2, H=1024, I=512, T=1200, zipf=1.1)


@pytest.mark.parametrize("mx", [False, True], ids=["general-scales", "pow2-scales"])
def test_every_tile_class_every_row(mx):
    cfg = SKEWED.scaled(mx=mx)
    _, _, rep = check_moe_rows(cfg, rows=None)
    cls = rep["classes"]
    # the routing must reach every class (full and partial 256-row tiles,
    # a 128-row tile, streaming tiles)
    for name in ("full256", "part256", "t128", "stream"):
        assert cls[name][1] > 0, (name, cls)


def test_headline_prefill_stratified():
    cfg = synth.C4_PREFILL
    _, _, rep = check_moe_rows(cfg, rows="stratified", sample_tokens=256, full_tokens=2)
    cls = rep["classes"]
    for name in ("full256", "part256", "t128", "stream"):
        assert cls[name][0] > 0, (name, cls)


def test_decode_batch_every_row():
    _, _, rep = check_moe_rows(synth.C4_DECODE, rows=None, sample_tokens=64, full_tokens=2)
    assert rep["rows"] == synth.C4_DECODE.T * synth.C4_DECODE.k


def test_512_experts_stratified():
    _, _, rep = check_moe_rows(synth.C3, rows="stratified", sample_tokens=128, full_tokens=2)
    assert rep["classes"]["t128"][0] > 0


def test_dense_mlp_M8192_as_one_expert():
    """The grouped path with E = 1 (every row in 256-row tiles, a 0-row
    remainder) on sampled rows of each 256-row tile position."""
    cfg = synth.MoE(seed=36, E=1, k=1, H=5120, I=17408, T=8192)
    rng = np.random.default_rng(8192)
    rows = np.unique(np.r_[0, 1, 255, 256, 4095, 4096, 8191, rng.choice(8192, 13, replace=False)])
    step(f"dense MLP M=8192 rows {rows.tolist()}")
    check_moe_rows(cfg, rows=rows, sample_tokens=64, full_tokens=4)
