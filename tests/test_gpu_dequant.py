"""tq_dequant_kv on the GPU against the oracle's dequantization to the
original space (K = R^T (gamma c[code]) for MSE keys, E4M3 values for FP8
keys, V = zero + scale * code), on identical cache bytes.

Bars: FP8 keys bit-exact in every output type (E4M3 values are exact in
fp16, bf16 and fp32).  MSE keys and values: within one unit in the last
place of the output type of the float64 result, plus the fp32 rounding of
the kernel's transform (4e-6 of the row's largest magnitude; the kernel
works in fp32, rounds once to the output type).  Rows outside the prefix,
and bytes between rows of a strided output, are untouched."""

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

D = 128
OUT = {"f16": (np.float16, 2.0 ** -10), "bf16": (None, 2.0 ** -7), "f32": (np.float32, 2.0 ** -23)}


def _torch_dtype(name):
    import torch

    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def _cache(preset, n, Hk, bs, seed, dtype="bf16", D=D):
    """Oracle-written cache of one sequence of n tokens in a shuffled pool."""
    rng = np.random.default_rng(seed)
    lay = O.layout(preset, D)
    c32, b32 = G.oracle_tables(lay)
    s = W.signs(seed, D)
    nbl = -(-n // bs)
    nb = nbl + 3
    table = rng.permutation(nb)[:nbl].astype(np.int32)
    cache = np.zeros((nb, bs, Hk, lay.slot_size_aligned), np.uint8)
    scale = np.exp(rng.uniform(np.log(0.25), np.log(8.0), (1, Hk, D)))
    K = O.widen(W.to_bits(rng.standard_normal((n, Hk, D)) * scale, dtype), dtype)
    V = O.widen(W.to_bits(rng.standard_normal((n, Hk, D)) * scale, dtype), dtype)
    slots = table[np.arange(n) // bs].astype(np.int64) * bs + np.arange(n) % bs
    if n:
        O.store(lay, K, V, slots, cache, s, c32, b32)
    return lay, cache, table, s, c32


def _gpu(preset, cache, table, n, s, out, stride_tokens=None, sentinel=None, D=D, block_layout="aos"):
    """cache: combined slots (converted to the SoA convention for block_layout "soa")."""
    import torch
    import quantized_decode_attention_tq_amd as tq

    lay_c = tq.layout_init(preset, D, block_layout)
    if block_layout == "soa":
        cache = O.soa_from_aos(O.layout(preset, D), cache)
    Hk = cache.shape[2]
    tab = G.gpu_tables(lay_c, s)
    dt = _torch_dtype(out)
    rows = stride_tokens or 1
    kb = torch.full((n, Hk * rows, D), float("nan") if sentinel is None else sentinel, dtype=dt, device="cuda")
    vb = kb.clone()
    ko, vo = kb[:, :Hk], vb[:, :Hk]  # token stride rows * Hk * D: strided rows of a larger buffer
    tq.dequant_kv(lay_c, torch.from_numpy(cache).cuda(), torch.from_numpy(table).cuda(), n, tab.signs,
                  tab.centroids, key_out=ko, value_out=vo)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(kb), f(vb)


def _check(got, want, out, exact=False):
    """got/want (n, Hk, D)."""
    if exact:
        np.testing.assert_array_equal(got, want)
        return
    _, rel = OUT[out]
    ulp = rel * np.maximum(np.abs(want), 2.0 ** -14)
    row = np.max(np.abs(want), axis=2, keepdims=True)
    err = np.abs(got - want)
    assert np.all(err <= ulp + 4e-6 * row), (err / (ulp + 4e-6 * row)).max()


def _oracle(lay, cache, table, n, s, c32):
    Hk = cache.shape[2]
    Ks, Vs = [], []
    for h in range(Hk):
        k, v = O.dequant_original_space(lay, cache, table, n, h, s, c32)
        Ks.append(k)
        Vs.append(v)
    return np.stack(Ks, 1), np.stack(Vs, 1)


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("out", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("n,Hk,bs", [(1, 8, 16), (300, 8, 16), (37, 3, 128), (129, 1, 64)])
def test_dequant_parity(preset, out, n, Hk, bs):
    G.log(f"dequant {preset} out={out} n={n} Hk={Hk} bs={bs}")
    lay, cache, table, s, c32 = _cache(preset, n, Hk, bs, seed=n + Hk)
    k, v = _gpu(preset, cache, table, n, s, out)
    kw, vw = _oracle(lay, cache, table, n, s, c32)
    _check(k, kw, out, exact=lay.key_fp8)
    _check(v, vw, out)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_3bit_nc"])
def test_dequant_into_strided_rows_touches_nothing_else(preset):
    """Output rows land every 3 * Hk heads of a larger buffer; the rest of
    the buffer keeps its sentinel."""
    n, Hk, bs = 70, 2, 32
    G.log(f"dequant strided {preset}")
    lay, cache, table, s, c32 = _cache(preset, n, Hk, bs, seed=9)
    k, v = _gpu(preset, cache, table, n, s, "f32", stride_tokens=3, sentinel=-7.0)
    kw, vw = _oracle(lay, cache, table, n, s, c32)
    _check(k[:, :Hk], kw, "f32", exact=lay.key_fp8)
    _check(v[:, :Hk], vw, "f32")
    assert np.all(k[:, Hk:] == -7.0) and np.all(v[:, Hk:] == -7.0)


def test_dequant_empty_prefix_is_a_no_op():
    import torch
    import quantized_decode_attention_tq_amd as tq

    lay_c = tq.layout_init("turboquant_4bit_nc")
    cache = torch.zeros((2, 16, 2, lay_c.slot_size_aligned), dtype=torch.uint8, device="cuda")
    ko = torch.full((4, 2, D), 3.0, device="cuda")
    vo = ko.clone()
    tab = tq.Tables(lay_c, W.signs(0))
    tq.dequant_kv(lay_c, cache, torch.zeros(1, dtype=torch.int32, device="cuda"), 0, tab.signs, tab.centroids,
                  key_out=ko, value_out=vo)
    torch.cuda.synchronize()
    assert bool((ko == 3.0).all()) and bool((vo == 3.0).all())


@pytest.mark.parametrize("preset", O.PRESETS)
def test_dequant_long_prefix_sampled(preset):
    """A 131072-token prefix of 8 KV heads in 128-token blocks (the long
    context shape), stored by the GPU: sampled tokens against the oracle
    on the same cache bytes, first and last tokens included."""
    import torch
    import quantized_decode_attention_tq_amd as tq

    n, Hk, bs = 131072, 8, 128
    G.log(f"dequant long prefix {preset}")
    rng = np.random.default_rng(77)
    lay = O.layout(preset, D)
    lay_c = tq.layout_init(preset)
    c32, _ = G.oracle_tables(lay)
    s = W.signs(5)
    tab = tq.Tables(lay_c, s)
    nb = n // bs
    table = rng.permutation(nb).astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(5)
    K = torch.randn((n, Hk, D), device="cuda", generator=g).to(torch.bfloat16)
    V = torch.randn((n, Hk, D), device="cuda", generator=g).to(torch.bfloat16)
    slots = torch.from_numpy(table[np.arange(n) // bs].astype(np.int64) * bs + np.arange(n) % bs).cuda()
    cache = torch.zeros(tq.kv_cache_shape(lay_c, nb, bs, Hk), dtype=torch.uint8, device="cuda")
    tq.store(lay_c, K, V, slots, cache, tab.signs, tab.centroids, tab.boundaries)
    ko, vo = tq.dequant_kv(lay_c, cache, torch.from_numpy(table).cuda(), n, tab.signs, tab.centroids,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    pick = np.concatenate([[0, n - 1], rng.integers(0, n, 62)])
    idx = torch.from_numpy(pick).cuda()
    k_np = ko[idx].cpu().numpy().astype(np.float64)
    v_np = vo[idx].cpu().numpy().astype(np.float64)
    blk = torch.from_numpy(table[pick // bs].astype(np.int64)).cuda()
    c_np = cache[blk, torch.from_numpy(pick % bs).cuda()].cpu().numpy()  # (samples, Hk, slot)
    R = O.rotation(np.asarray(s, np.float64)) if O.needs_rotation(lay) else None
    for i in range(len(pick)):
        Kd, Vd = O.decode_slots(lay, c_np[i], c32, R)
        if not lay.key_fp8:
            Kd = Kd @ R
        _check(k_np[i][None], Kd[None], "f32", exact=lay.key_fp8)
        _check(v_np[i][None], Vd[None], "f32")


@pytest.mark.parametrize("i", range(36))
def test_dequant_random_configurations(i):
    """Seeded random configurations: preset (each three times), head_dim,
    KV heads, block size, block convention, prefix length (one-token and
    block-edge prefixes included), output dtype; the parity bars above."""
    rng = np.random.default_rng(3000 + i)
    preset = list(O.PRESETS)[i % len(O.PRESETS)]
    d = 256 if rng.random() < 0.25 else 128
    Hk = int(rng.choice([1, 2, 3, 4, 8, 16]))
    bs = int(rng.choice([16, 32, 64, 128]))
    n = int(rng.choice([1, bs - 1, bs, bs + 1, int(rng.integers(2, 700)), int(rng.integers(2, 700))]))
    out = str(rng.choice(["f16", "bf16", "f32"]))
    layout = "soa" if rng.random() < 0.4 and (Hk <= 8 or Hk % 8 == 0) else "aos"
    G.log(f"dequant random {i}: {preset} D={d} Hk={Hk} bs={bs} n={n} {out} {layout}")
    lay, cache, table, s, c32 = _cache(preset, n, Hk, bs, seed=4000 + i, D=d)
    k, v = _gpu(preset, cache, table, n, s, out, D=d, block_layout=layout)
    kw, vw = _oracle(lay, cache, table, n, s, c32)
    _check(k, kw, out, exact=lay.key_fp8)
    _check(v, vw, out)
