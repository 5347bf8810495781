"""tq_decode_attention on the GPU against the oracle's exact softmax attention
over the dequantized cache: per (sequence, query head) max |o - o_ref| /
max |o_ref| <= 5e-3 (fp32 output), LSE within 5e-3.  Checked on identical
cache bytes (written by the oracle) and end to end (GPU store + GPU decode).
"""

import math

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

ALL_ROWS = None


def _rows(w):
    return [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]


def _small(preset, lens, Hq, Hk, bs, dtype="bf16", dist="normal_chscale", seed=31):
    return W.Workload("t", preset, len(lens), Hq, Hk, bs, dtype, dist, seed=seed, lens=tuple(lens), pool_factor=1.5,
                      chscale_range=(0.5, 4.0), outliers=4, outlier_scale=8.0)


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("S", [1, 3, 8])
def test_decode_parity_identical_bytes(preset, S):
    w = _small(preset, [1, 37, 300, 16], Hq=8, Hk=2, bs=16)
    G.log(f"decode {preset} S={S} lens={w.lens}")
    c = G.DecodeCase(w)
    import torch

    cache = torch.from_numpy(c.cache_o).cuda()
    out, lse = c.gpu_decode(cache, S)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_decode_end_to_end_block_sizes(preset, bs):
    w = _small(preset, [bs - 1, bs, bs + 1, 3 * bs + 5, 0], Hq=4, Hk=2, bs=bs, seed=40 + bs)
    G.log(f"decode e2e {preset} bs={bs} lens={w.lens}")
    c = G.DecodeCase(w)
    cache = c.gpu_store_all()
    out, lse = c.gpu_decode(cache, 4)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("batch", [24, 48])
def test_decode_heads_per_workgroup_modes(preset, batch):
    """Enough (sequence, split) units select 2 (24 sequences) or 4 (48
    sequences) KV heads per workgroup with 8 KV heads and 8 splits."""
    rng = np.random.default_rng(batch)
    lens = [int(x) for x in rng.integers(1, 160, batch)]
    lens[0], lens[1] = 0, 16
    w = _small(preset, lens, Hq=16, Hk=8, bs=16, seed=70 + batch)
    G.log(f"decode modes {preset} B={batch}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 8)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("g", [1, 2, 4, 5, 8, 16, 20])
def test_decode_gqa_groups(g):
    w = _small("turboquant_k3v4_nc", [70, 129], Hq=2 * g, Hk=2, bs=32, seed=60 + g)
    G.log(f"decode gqa g={g}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 2)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


def test_decode_tiny_workload_and_out_dtypes():
    """The tiny workload (4bit_nc, 256 tokens, GQA 2, fp16, sequential
    blocks): store all 256 tokens, decode one query."""
    import torch

    w = W.WORKLOADS["tiny"]
    G.log("decode tiny")
    c = G.DecodeCase(w)
    cache = c.gpu_store_all()
    ref, rlse = c.oracle_decode()
    for S in (1, 4, 16, 40):
        out, lse = c.gpu_decode(cache, S)
        G.check_decode(out, lse, ref, rlse, _rows(w))
    for dt in (torch.float16, torch.bfloat16):
        out, lse = c.gpu_decode(cache, 4, out_dtype=dt)
        tol = 2.0 ** -8 if dt == torch.bfloat16 else 2.0 ** -11
        for b, h in _rows(w):
            err = np.max(np.abs(out[b, h] - ref[b, h])) / np.max(np.abs(ref[b, h]))
            assert err <= G.DECODE_RTOL + tol, (dt, err)


def test_decode_special_inputs():
    """Zero query: uniform attention -> mean of the values.  Peaked query:
    output follows the one matching token."""
    import torch

    w = _small("turboquant_4bit_nc", [50, 77], Hq=4, Hk=2, bs=16, seed=5)
    c = G.DecodeCase(w)
    c.qbits[0] = 0
    G.log("decode special inputs")
    c.q = G.dev16(c.qbits, w.dtype)
    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 2)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))
    _, Vd = O.gather_sequence(c.lay, c.cache_o, c.table[0], 50, 0, c.c32)
    np.testing.assert_allclose(out[0, 0], Vd.mean(axis=0), rtol=2e-3, atol=2e-3 * np.abs(Vd).max())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,S,rows", [
    ("llama8b", 8, [(0, 0), (7, 13), (31, 31)]),
    ("longctx", 32, [(0, 0), (3, 39), (2, 17)]),
    ("qwen32b", 8, [(0, 0), (40, 63), (63, 9)]),
])
def test_decode_full_size_sampled(name, S, rows):
    """Full-size workloads in the benchmark's launch configuration: the GPU
    stores and decodes everything; the oracle recomputes sampled rows from
    the raw inputs."""
    w = W.WORKLOADS[name]
    G.log(f"decode full-size {name} S={S}: generating inputs")
    c = G.DecodeCase(w, need_oracle_cache=False)
    G.log(f"decode full-size {name}: store")
    cache = c.gpu_store_all()
    G.log(f"decode full-size {name}: decode")
    out, lse = c.gpu_decode(cache, S)
    assert np.all(np.isfinite(out))
    G.log(f"decode full-size {name}: oracle rows {rows}")
    res = c.oracle_decode_rows_from_inputs(rows)
    for (b, hq), (ro, rl) in res.items():
        err = np.max(np.abs(out[b, hq] - ro)) / np.max(np.abs(ro))
        assert err <= G.DECODE_RTOL, (b, hq, err)
        assert abs(lse[b, hq] - rl) <= G.LSE_ATOL * max(1.0, abs(rl))


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_3bit_nc"])
@pytest.mark.parametrize("S", [1, 4, 32])
def test_decode_ragged_lengths_balanced_units(preset, S):
    """Very uneven lengths: the work units are spread in proportion to
    length, empty sequences get none (o = 0, lse = -inf)."""
    w = _small(preset, [1, 2000, 17, 0, 700, 40], Hq=4, Hk=2, bs=16, seed=90 + S)
    G.log(f"decode ragged {preset} S={S}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), S)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset,Hk,g", [("turboquant_k3v4_nc", 1, 2), ("turboquant_k8v4", 8, 4),
                                         ("turboquant_3bit_nc", 8, 5)])
def test_decode_many_sequences(preset, Hk, g):
    """More than 64 sequences: the unit search scans the lengths in several
    64-wide passes (8 KV heads: the fixed-geometry kernels)."""
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(0, 90, 150)]
    w = _small(preset, lens, Hq=Hk * g, Hk=Hk, bs=32, seed=12)
    G.log(f"decode 150 sequences {preset} Hk={Hk} g={g}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 3)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset,lens,S", [
    ("turboquant_k8v4", [1200, 40, 700, 16, 0, 333, 1600, 90] * 4, 8),
    ("turboquant_3bit_nc", [2048, 17, 900, 1500, 64, 300, 1, 1100] * 3, 8),
    ("turboquant_k3v4_nc", [4000, 100, 2500, 700] * 2, 32),
])
def test_ragged_units_cover_every_tile(preset, lens, S):
    """Ragged batches on the fixed-geometry kernels (8 KV heads): every unit of
    the length-balanced split is computed and merged.  A workspace filled
    with 0xFF (NaN partial rows) leaves any unit that no workgroup wrote as
    NaN in the output."""
    w = _small(preset, lens, Hq=8 * 4, Hk=8, bs=16, seed=90 + S)
    G.log(f"ragged pairing {preset} B={len(lens)} S={S}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode_two_stage(torch.from_numpy(c.cache_o).cuda(), S, workspace_fill=0xFF)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))


@pytest.mark.parametrize("preset,Hk,g", [
    ("turboquant_4bit_nc", 1, 4),     # one head: 8 phase waves
    ("turboquant_k8v4", 3, 2),        # contiguous group of 3 heads, 2 phases
    ("turboquant_k3v4_nc", 16, 2),    # groups of 8 heads, 16-byte aligned row pieces
    ("turboquant_4bit_nc", 12, 1),    # groups of 6 heads, misaligned row pieces
    ("turboquant_k8v4", 12, 3),       # groups of 4 heads, aligned (196-byte slots), 2 phases
])
def test_decode_head_groupings(preset, Hk, g):
    w = _small(preset, [45, 130, 16], Hq=Hk * g, Hk=Hk, bs=32, seed=100 + Hk)
    G.log(f"decode groupings {preset} Hk={Hk} g={g}")
    c = G.DecodeCase(w)
    import torch

    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 2)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))



@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("S", [1, 8])
def test_split_entry_points_match_single_call(preset, S):
    """tq_decode_stage1 + tq_decode_stage2 on a workspace holding garbage give
    what tq_decode_attention gives (the same two launches), within the oracle
    bar, including sequences of length 0."""
    w = _small(preset, [0, 1, 37, 300, 16, 1000, 0, 129], Hq=8, Hk=2, bs=16, seed=90 + S)
    G.log(f"split entry points {preset} S={S} lens={w.lens}")
    c = G.DecodeCase(w)
    import torch

    cache = torch.from_numpy(c.cache_o).cuda()
    out2, lse2 = c.gpu_decode_two_stage(cache, S, workspace_fill=0x7F)
    out1, lse1 = c.gpu_decode(cache, S)
    ref, rlse = c.oracle_decode()
    G.check_decode(out2, lse2, ref, rlse, _rows(w))
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("factor", [3e5, 1e9, 1e-7])
def test_decode_query_magnitudes(preset, factor):
    """bf16 queries far outside fp16 range (and far below its normal range):
    each query head's fp16 operand is scaled by a power of two, so the result
    still meets the bar (huge queries give one-hot attention, tiny ones
    near-uniform attention)."""
    import torch

    w = _small(preset, [40, 300, 16], Hq=8, Hk=2, bs=16, seed=77)
    c = G.DecodeCase(w)
    q = O.widen(c.qbits, "bf16") * factor
    c.qbits = W.to_bits(q, "bf16")
    c.q = G.dev16(c.qbits, "bf16")
    G.log(f"decode query x{factor:g} {preset}")
    out, lse = c.gpu_decode(torch.from_numpy(c.cache_o).cuda(), 3)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))
