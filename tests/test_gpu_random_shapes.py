"""Seeded random decode configurations against the oracle: preset, head_dim,
KV heads, GQA group, block size, block convention, sequence lengths (empty
and one-token sequences included), split count, sliding window, sinks and
input / output dtypes drawn per case, so that combinations no hand-written
case names still meet the store and decode bars.  Each case stores every
sequence on the GPU, checks the stored slots against the oracle's encoding
of the same rows, then decodes every query head and checks it against the
oracle's attention over the same cache bytes."""

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

PRESETS = list(O.PRESETS)
N_CASES = 96


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    preset = PRESETS[i % len(PRESETS)]  # every preset eight times
    D = 256 if rng.random() < 0.2 else 128
    Hk = int(rng.choice([1, 2, 3, 4, 8, 16]))
    g = int(rng.choice([1, 2, 4, 5, 8, 16]))
    while Hk * g > 64:
        g //= 2
    g = max(g, 1)
    layout = "soa" if rng.random() < 0.3 and (Hk <= 8 or Hk % 8 == 0) else "aos"
    bs = int(rng.choice([16, 32, 64, 128]))
    B = int(rng.integers(1, 6))
    lens = rng.integers(0, 1100, B)
    specials = [0, 1, 16, bs, bs + 1, 17]
    for j in range(B):
        if rng.random() < 0.3:
            lens[j] = specials[int(rng.integers(len(specials)))]
    if lens.max() == 0:
        lens[0] = 5
    S = int(rng.integers(1, 33))
    window = int(rng.integers(1, 700)) if rng.random() < 0.3 else 0
    sinks = rng.uniform(-2.0, 6.0, Hk * g) if rng.random() < 0.3 else None
    dtype = "bf16" if rng.random() < 0.6 else "f16"
    out = str(rng.choice(["f32", "f16", "bf16"]))
    w = W.Workload(f"rand{i}", preset, B, Hk * g, Hk, bs, dtype, "normal_chscale", seed=500 + i,
                   lens=tuple(int(x) for x in lens), pool_factor=1.5, chscale_range=(0.5, 4.0), head_dim=D)
    return w, layout, S, window, sinks, out


@pytest.mark.timeout(240)
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode_configuration(i):
    import torch

    w, layout, S, window, sinks, out = _draw(i)
    G.log(f"random case {i}: {w.preset} D={w.head_dim} Hk={w.num_kv_heads} Hq={w.num_q_heads} bs={w.block_size} "
          f"{layout} lens={list(w.lens)} S={S} window={window} sinks={sinks is not None} {w.dtype}->{out}")
    c = G.DecodeCase(w, need_oracle_cache=False, block_layout=layout)
    cache = c.gpu_store_all()
    got = c.as_oracle_cache(cache.cpu().numpy())

    # store: every stored slot against the oracle's encoding of its row
    R = O.rotation(c.signs.astype(np.float64)) if O.needs_rotation(c.lay) else None
    gots, wants, keys, vals = [], [], [], []
    for b in range(w.batch):
        L = int(c.lens[b])
        if L == 0:
            continue
        slots = W.slot_mapping_for_sequence(w, b, c.table, c.lens)
        for hk in range(w.num_kv_heads):
            k = O.widen(c.K[b][:, hk], w.dtype)
            v = O.widen(c.V[b][:, hk], w.dtype)
            gots.append(got[slots // w.block_size, slots % w.block_size, hk])
            wants.append(O.encode_slots(c.lay, k, v, R, c.c32, c.b32))
            keys.append(k)
            vals.append(v)
    G.compare_slots(c.lay, np.concatenate(gots), np.concatenate(wants), np.concatenate(keys), c.signs, c.c32, c.b32,
                    np.concatenate(vals), min_allowed=2)

    # decode: every query head against the oracle on the same bytes
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]
    o, lse = c.gpu_decode(cache, S, out_dtype=dt, sliding_window=window, sinks=sinks)
    ref, rlse = c.oracle_decode(cache=got, sliding_window=window, sinks=sinks)
    rows = [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
    worst = G.check_decode(o, lse, ref, rlse, rows)
    G.log(f"random case {i}: worst row error {worst:.2e}")
