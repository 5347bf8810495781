"""tq_decode_attention_noalloc (the entry point that allocates nothing and
keeps its stage-1 scratch in the library's device array) against
tq_decode_attention on the same inputs: identical output and LSE (the same
kernels and launch plan), and both within the oracle bar.  Two calls in a
row, the second smaller, so that what the first leaves in the shared scratch
cannot leak into the second; then a case near the scratch limit."""

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _small(preset, lens, Hq, Hk, bs, seed):
    return W.Workload("t", preset, len(lens), Hq, Hk, bs, "bf16", "normal_chscale", seed=seed, lens=tuple(lens),
                      pool_factor=1.5, chscale_range=(0.5, 4.0), outliers=4, outlier_scale=8.0)


def _both(c, S, sinks=None, window=0):
    import torch
    import quantized_decode_attention_tq_amd as tq

    cache = torch.from_numpy(c.cache_o).cuda()
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    B, Hq = c.q.shape[:2]
    out = torch.full((B, Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    tq.decode_noalloc(c.lay_c, c.q, cache, c.bt, c.sl, c.tab.signs, c.tab.centroids, c.scale, S, out, lse,
                      sliding_window=window, sinks=sk)
    ref_out, ref_lse = tq.decode(c.lay_c, c.q, cache, c.bt, c.sl, c.tab.signs, c.tab.centroids, c.scale, S,
                                 out_dtype=torch.float32, sliding_window=window, sinks=sk)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out.cpu().numpy().astype(np.float64), ref_lse.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_noalloc_matches_workspace_entry_two_calls(preset):
    rows = lambda w: [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
    # first call: 6 ragged sequences (one empty), 8 splits
    w1 = _small(preset, [300, 1000, 17, 0, 700, 40], Hq=8, Hk=2, bs=16, seed=3)
    G.log(f"noalloc {preset} call 1 lens={w1.lens}")
    c1 = G.DecodeCase(w1)
    out, lse, rout, rlse = _both(c1, 8)
    np.testing.assert_array_equal(out, rout)
    np.testing.assert_array_equal(lse, rlse)
    ref, reflse = c1.oracle_decode()
    G.check_decode(out, lse, ref, reflse, rows(w1))
    # second call: fewer, shorter sequences, with a window and sinks
    w2 = _small(preset, [33, 5], Hq=4, Hk=1, bs=32, seed=4)
    G.log(f"noalloc {preset} call 2 lens={w2.lens}")
    c2 = G.DecodeCase(w2)
    sinks = np.array([0.5, -1.0, 2.0, 0.0])
    out, lse, rout, rlse = _both(c2, 3, sinks=sinks, window=20)
    np.testing.assert_array_equal(out, rout)
    np.testing.assert_array_equal(lse, rlse)
    ref, reflse = c2.oracle_decode(sliding_window=20, sinks=sinks)
    G.check_decode(out, lse, ref, reflse, rows(w2))


def test_noalloc_near_the_scratch_limit():
    """64 sequences x 64 query heads with 8 splits: a workspace of ~17 MB of
    the 32 MiB scratch."""
    import quantized_decode_attention_tq_amd as tq

    rng = np.random.default_rng(8)
    lens = [int(x) for x in rng.integers(1, 120, 64)]
    w = _small("turboquant_3bit_nc", lens, Hq=64, Hk=8, bs=16, seed=9)
    assert tq.decode_workspace_bytes(64, 64, 128, 8) > tq.NOALLOC_SCRATCH_BYTES // 2
    G.log("noalloc 64 x 64 heads")
    c = G.DecodeCase(w)
    out, lse, rout, rlse = _both(c, 8)
    np.testing.assert_array_equal(out, rout)
    np.testing.assert_array_equal(lse, rlse)
    rows = [(b, h) for b in (0, 31, 63) for h in range(64)]
    ref, reflse = c.oracle_decode(rows=rows)
    G.check_decode(out, lse, ref, reflse, rows)
