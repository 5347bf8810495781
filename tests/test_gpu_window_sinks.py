"""Sliding-window decode and attention sinks on the GPU against the oracle
(the oracle's window_start / attend readings): the decode bar (5e-3 max
relative error per (sequence, query head), LSE 5e-3) on identical cache
bytes, for windows shorter than, equal to and longer than the sequences,
starting inside a tile, and for sinks below, near and above the scores,
including empty sequences (o = 0, lse = the sink)."""

import math

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _small(preset, lens, Hq, Hk, bs, seed=31):
    return W.Workload("t", preset, len(lens), Hq, Hk, bs, "bf16", "normal_chscale", seed=seed, lens=tuple(lens),
                      pool_factor=1.5, chscale_range=(0.5, 4.0), outliers=4, outlier_scale=8.0)


def _rows(w):
    return [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("window", [1, 7, 16, 50, 129, 4000])
def test_sliding_window(preset, window):
    import torch

    w = _small(preset, [1, 20, 130, 0, 400, 50], Hq=8, Hk=2, bs=32, seed=60 + window)
    G.log(f"window {preset} W={window}")
    c = G.DecodeCase(w)
    cache = torch.from_numpy(c.cache_o).cuda()
    for S in (1, 4):
        out, lse = c.gpu_decode(cache, S, sliding_window=window)
        ref, rlse = c.oracle_decode(sliding_window=window)
        G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_k3v4_nc", "turboquant_2bit_nc"])
def test_sinks(preset):
    import torch

    w = _small(preset, [0, 1, 37, 300, 16], Hq=8, Hk=2, bs=16, seed=70)
    G.log(f"sinks {preset}")
    c = G.DecodeCase(w)
    cache = torch.from_numpy(c.cache_o).cuda()
    ref0, rlse0 = c.oracle_decode()
    finite = rlse0[np.isfinite(rlse0)]
    # per head: far below, near the typical LSE, above it
    sinks = np.array([-40.0, -2.0, 0.0, 1.0, float(np.median(finite)), float(finite.max()) + 3.0, 5.0, -np.inf],
                     np.float32)
    for S in (1, 8):
        out, lse = c.gpu_decode(cache, S, sinks=sinks)
        ref, rlse = c.oracle_decode(sinks=sinks)
        # empty sequences: o = 0 and lse = the sink (-inf for the head without one)
        assert np.all(out[0] == 0)
        np.testing.assert_allclose(lse[0], sinks.astype(np.float64), rtol=0, atol=0)
        G.check_decode(out, lse, ref, rlse, [(b, h) for b in range(1, w.batch) for h in range(w.num_q_heads)])


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_3bit_nc"])
def test_window_and_sinks_through_the_split_entry_points(preset):
    """stage 1 takes the window, stage 2 the sinks: the same result as the
    single call, and the oracle's."""
    import torch

    w = _small(preset, [0, 5, 70, 1000, 33], Hq=4, Hk=1, bs=64, seed=80)
    G.log(f"window+sinks split {preset}")
    c = G.DecodeCase(w)
    cache = torch.from_numpy(c.cache_o).cuda()
    sinks = np.array([0.5, -1.0, 3.0, 0.0], np.float32)
    out2, lse2 = c.gpu_decode_two_stage(cache, 4, workspace_fill=0x7F, sliding_window=100, sinks=sinks)
    out1, lse1 = c.gpu_decode(cache, 4, sliding_window=100, sinks=sinks)
    ref, rlse = c.oracle_decode(sliding_window=100, sinks=sinks)
    G.check_decode(out2, lse2, ref, rlse, _rows(w))
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


@pytest.mark.parametrize("block_layout", ["aos", "soa"])
def test_window_on_soa_and_packed_pairs(block_layout):
    """Windows starting in the first or second tile of a packed pair (GQA
    group <= 8, MSE keys), in both block conventions."""
    import torch

    w = _small("turboquant_k3v4_nc", [200, 201, 215, 230, 17], Hq=16, Hk=2, bs=16, seed=90)
    G.log(f"window packed {block_layout}")
    c = G.DecodeCase(w, block_layout=block_layout)
    cache = torch.from_numpy(c.oracle_cache_bytes()).cuda()
    for window in (33, 40, 48, 63):
        out, lse = c.gpu_decode(cache, 2, sliding_window=window)
        ref, rlse = c.oracle_decode(sliding_window=window)
        G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.timeout(600)
def test_window_and_sinks_full_size_sampled():
    """The long-context workload (4 x 131072 tokens) with an 8192-token
    window and per-head sinks, in the benchmark's launch configuration;
    sampled rows recomputed by the oracle from the raw inputs."""
    import torch

    w = W.WORKLOADS["longctx"]
    G.log("window + sinks longctx")
    c = G.DecodeCase(w, need_oracle_cache=False)
    cache = c.gpu_store_all()
    rng = np.random.default_rng(3)
    sinks = rng.uniform(-2.0, 6.0, w.num_q_heads).astype(np.float32)
    out, lse = c.gpu_decode(cache, 32, sliding_window=8192, sinks=sinks)
    rows = [(b, int(h)) for b in range(w.batch) for h in rng.integers(0, w.num_q_heads, 3)]
    res = c.oracle_decode_rows_from_inputs(rows, sliding_window=8192, sinks=sinks)
    ref = np.zeros_like(out)
    rlse = np.zeros_like(lse)
    for (b, h), (o, l) in res.items():
        ref[b, h], rlse[b, h] = o, l
    G.check_decode(out, lse, ref, rlse, rows)
