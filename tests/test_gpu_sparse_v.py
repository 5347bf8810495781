"""The opt-in sparse-V gate on the GPU against exact attention computed by
the oracle on identical cache bytes.  Per (sequence, query head) and dim:
|o - o_exact| <= bound + 5e-3 max |o_exact|, where bound is the oracle's
value mass of the tokens the gate may drop (exp(s - max) below the gate,
taken 10% wider to cover the kernel's fp16 scores); the lse is the exact
one.  The gate fires on these inputs (the output moves from the exact
decode)."""

import math

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

GATE = 1e-3


def _w(preset, lens, Hq, Hk, bs, seed, D=128):
    return W.Workload("sv", preset, len(lens), Hq, Hk, bs, "bf16", "normal_chscale", seed=seed, lens=tuple(lens),
                      pool_factor=1.5, chscale_range=(0.5, 4.0), head_dim=D)


def _check_gated(c, out, lse, sliding_window=0, sinks=None):
    w = c.w
    q = O.widen(c.qbits, w.dtype)
    R = O.rotation(c.signs.astype(np.float64)) if O.needs_rotation(c.lay) else None
    g = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        L = int(c.lens[b])
        f = O.window_start(L, sliding_window)
        for hk in range(w.num_kv_heads):
            K, V = O.gather_sequence(c.lay, c.cache_o, c.table[b], L, hk, c.c32, R)
            for hq in range(hk * g, (hk + 1) * g):
                qq = q[b, hq] if c.lay.key_fp8 else R @ q[b, hq]
                sink = -math.inf if sinks is None else float(np.float32(sinks[hq]))
                ox, lx = O.attend(qq, K[f:L], V[f:L], c.scale, sink)
                _, _, bound = O.attend_sparse_v(qq, K[f:L], V[f:L], c.scale, GATE * 1.1, sink)
                tol = G.DECODE_RTOL * max(np.max(np.abs(ox)), 1e-30)
                err = np.abs(out[b, hq] - ox)
                assert np.all(err <= bound + tol), (b, hq, float((err - bound).max()), tol)
                if lx == -math.inf:
                    assert lse[b, hq] == -math.inf and np.all(out[b, hq] == 0)
                else:
                    assert abs(lse[b, hq] - lx) <= G.LSE_ATOL * max(1.0, abs(lx)), (b, hq)


def _run(w, S, sliding_window=0, sinks=None):
    import torch

    c = G.DecodeCase(w)
    cache = torch.from_numpy(c.cache_o).cuda()
    out, lse = c.gpu_decode(cache, S, sliding_window=sliding_window, sinks=sinks, value_gate=GATE)
    _check_gated(c, out, lse, sliding_window, sinks)
    exact, _ = c.gpu_decode(cache, S, sliding_window=sliding_window, sinks=sinks)
    assert not np.array_equal(out, exact), "the gate never fired"


@pytest.mark.parametrize("preset", O.PRESETS)
def test_sparse_v_gate_within_bound(preset):
    """GQA 4 (MSE keys: two tiles scored packed), ragged lengths incl. 0."""
    w = _w(preset, [1, 37, 600, 2000, 0], 8, 2, 16, seed=5)
    G.log(f"sparse-V {preset} lens={w.lens}")
    _run(w, 4)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_3bit_nc", "turboquant_3bit_lm"])
def test_sparse_v_gate_wide_groups(preset):
    """GQA 16: MSE keys take two tiles per wave one at a time, FP8 keys one."""
    w = _w(preset, [900, 1500], 32, 2, 32, seed=6)
    G.log(f"sparse-V wide groups {preset}")
    _run(w, 3)


def test_sparse_v_gate_with_window_and_sinks():
    w = _w("turboquant_k3v4_nc", [300, 2500, 40], 8, 2, 16, seed=7)
    G.log("sparse-V with window + sinks")
    _run(w, 4, sliding_window=1000, sinks=np.linspace(-2.0, 3.0, 8))


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_3bit_lm"])
def test_sparse_v_gate_head256(preset):
    w = _w(preset, [700, 1300], 8, 2, 16, seed=8, D=256)
    G.log(f"sparse-V D=256 {preset}")
    _run(w, 2)


@pytest.mark.timeout(240)
@pytest.mark.parametrize("i", range(0, 96, 4))
def test_gate_on_random_configurations(i):
    """The gated kernels on the seeded random configurations of the random
    parity suite (every fourth: each preset twice, both block conventions,
    ragged lengths, windows, sinks): the same bound against exact attention
    on the oracle's cache bytes."""
    import torch

    from test_gpu_random_shapes import _draw

    w, layout, S, window, sinks, _ = _draw(i)
    G.log(f"gated random case {i}: {w.preset} D={w.head_dim} Hk={w.num_kv_heads} Hq={w.num_q_heads} "
          f"bs={w.block_size} {layout} lens={list(w.lens)} S={S} window={window} sinks={sinks is not None}")
    c = G.DecodeCase(w, block_layout=layout)
    cache = torch.from_numpy(c.oracle_cache_bytes()).cuda()
    out, lse = c.gpu_decode(cache, S, sliding_window=window, sinks=sinks, value_gate=GATE)
    _check_gated(c, out, lse, window, sinks)
