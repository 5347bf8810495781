"""The SoA block convention on the GPU: store, decode attention and dequant
of an SoA cache against the oracle (whose SoA bytes are the combined slots
permuted block by block, oracle.soa_from_aos), to the same bars as the
combined-slot tests; and, since only the addressing differs, SoA results
bit-identical to the combined-slot results on the same logical cache."""

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


def _same_plan(lay, Hk):
    """Whether the stage-1 launch plans of the two conventions agree (then
    the arithmetic, hence every bit, is the same).  Restates the host plan
    rule: a tile image of spt 1 KB LDS slots (combined slots: ceil(G * slot
    / 64), plus a chunk of slack per row piece for groups of 8 of more heads;
    SoA: 16 image rows of G data rows plus a 16-byte pad, then the records,
    each part rounded up to whole slots); P = min(8 / G, 2) phase waves; MSE keys take
    two tiles per wave when P * spt <= 20; ring depth = 52 // (P * tpw * spt)
    clamped to 2..4."""
    G = min(Hk, 8)
    P = 1 if G >= 8 else min(8 // G, 2)
    data, _, nf = O.soa_geometry(lay, 16, G)
    if Hk <= 8:
        spt_a = -(-G * lay.slot_size_aligned // 64)
    else:
        spt_a = -(-16 * ((G * lay.slot_size_aligned + 30) // 16) // 64)
    spt_s = -(-(G * data + 16) // 64) + -(-G * 2 * nf // 64)

    def plan(spt):
        tpw = 2 if (not lay.key_fp8 and P * spt <= 20) else 1
        return tpw, min(max(52 // (P * tpw * spt), 2), 4)

    return plan(spt_a) == plan(spt_s)


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("Hk,bs", [(3, 16), (8, 32), (16, 128)])
def test_soa_store_parity(preset, Hk, bs):
    """GPU store into an SoA cache = the oracle's store, permuted: compared in
    the combined view (codes near a boundary, norms 1e-3, the rest exact),
    every byte outside the written rows keeps its sentinel."""
    import torch
    import quantized_decode_attention_tq_amd as tq

    seed, N, sentinel = 20 + Hk, 700, 0x5A
    G.log(f"soa store {preset} Hk={Hk} bs={bs}")
    K, V, slots, nb = W.store_inputs(num_tokens=N, num_kv_heads=Hk, block_size=bs, seed=seed, dtype="bf16")
    nb += 1
    slots[::11] = -1
    lay = O.layout(preset, G.D)
    lay_c = tq.layout_init(preset, G.D, "soa")
    signs = W.signs(seed)
    c32, b32 = G.oracle_tables(lay)
    tab = G.gpu_tables(lay_c, signs)
    shape = (nb, bs, Hk, lay.slot_size_aligned)
    cache = torch.full(shape, sentinel, dtype=torch.uint8, device="cuda")
    tq.store(lay_c, G.dev16(K, "bf16"), G.dev16(V, "bf16"), torch.from_numpy(slots).cuda(), cache, tab.signs,
             tab.centroids, tab.boundaries)
    torch.cuda.synchronize()
    got = O.aos_from_soa(lay, cache.cpu().numpy())
    want = np.full(shape, sentinel, np.uint8)
    O.store_rows(lay, O.widen(K, "bf16"), O.widen(V, "bf16"), slots, want, signs, c32, b32)
    written = np.zeros(shape[:3], bool)
    keep = slots >= 0
    written[slots[keep] // bs, slots[keep] % bs] = True
    np.testing.assert_array_equal(got[~written], want[~written])
    rg = got[slots[keep] // bs, slots[keep] % bs].reshape(-1, lay.slot_size_aligned)
    rw = want[slots[keep] // bs, slots[keep] % bs].reshape(-1, lay.slot_size_aligned)
    G.compare_slots(lay, rg, rw, O.widen(K[keep], "bf16").reshape(-1, G.D), signs, c32, b32,
                    O.widen(V[keep], "bf16").reshape(-1, G.D))


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("Hk,g,bs,S", [(2, 4, 16, 3), (8, 4, 64, 8), (1, 5, 32, 2), (3, 2, 128, 1), (16, 2, 32, 4)])
def test_soa_decode_parity_identical_bytes(preset, Hk, g, bs, S):
    """Decode over the oracle's cache in the SoA convention: against the
    oracle, and bit-identical to the combined-slot decode of the same cache
    when both launch plans agree (one KV head with 3-bit keys takes an extra
    LDS slot per tile in SoA, which changes the plan)."""
    import torch

    w = _small(preset, [1, bs - 1, 3 * bs + 7, 0, 300], Hq=Hk * g, Hk=Hk, bs=bs, seed=50 + Hk + bs)
    G.log(f"soa decode {preset} Hk={Hk} g={g} bs={bs} S={S}")
    c = G.DecodeCase(w, block_layout="soa")
    out, lse = c.gpu_decode(torch.from_numpy(c.oracle_cache_bytes()).cuda(), S)
    ref, rlse = c.oracle_decode()
    G.check_decode(out, lse, ref, rlse, _rows(w))
    if _same_plan(c.lay, Hk):
        a = G.DecodeCase(w, need_oracle_cache=False)
        out_a, lse_a = a.gpu_decode(torch.from_numpy(c.cache_o).cuda(), S)
        np.testing.assert_array_equal(out, out_a)
        np.testing.assert_array_equal(lse, lse_a)


@pytest.mark.parametrize("preset", O.PRESETS)
def test_soa_store_then_decode(preset):
    """GPU store into an SoA cache, then GPU decode of it, against the oracle
    on the inputs (end to end)."""
    w = _small(preset, [17, 200, 64, 1], Hq=16, Hk=8, bs=16, seed=77)
    G.log(f"soa e2e {preset}")
    c = G.DecodeCase(w, block_layout="soa")
    cache = c.gpu_store_all()
    out, lse = c.gpu_decode(cache, 4)
    ref, rlse = c.oracle_decode(cache=c.as_oracle_cache(cache.cpu().numpy()))
    G.check_decode(out, lse, ref, rlse, _rows(w))
    ref2, rlse2 = c.oracle_decode()  # the oracle's own store: codes may differ next to a boundary only
    G.check_decode(out, lse, ref2, rlse2, _rows(w))


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("Hk,bs", [(3, 16), (8, 128)])
def test_soa_dequant_bit_identical_to_combined(preset, Hk, bs):
    """Dequant of an SoA cache equals the dequant of the same cache in
    combined slots, bit for bit, in every output type (the combined path is
    checked against the oracle by the dequant tests)."""
    import torch
    import quantized_decode_attention_tq_amd as tq

    rng = np.random.default_rng(Hk + bs)
    lay = O.layout(preset, G.D)
    n = 5 * bs - 3
    nb = -(-n // bs) + 2
    table = rng.permutation(nb)[: -(-n // bs)].astype(np.int32)
    c32, b32 = G.oracle_tables(lay)
    s = W.signs(3)
    cache = np.zeros((nb, bs, Hk, lay.slot_size_aligned), np.uint8)
    K = O.widen(W.to_bits(rng.standard_normal((n, Hk, G.D)) * 2.0, "bf16"), "bf16")
    V = O.widen(W.to_bits(rng.standard_normal((n, Hk, G.D)), "bf16"), "bf16")
    slots = table[np.arange(n) // bs].astype(np.int64) * bs + np.arange(n) % bs
    O.store_rows(lay, K, V, slots, cache, s, c32, b32)
    G.log(f"soa dequant {preset} Hk={Hk} bs={bs}")
    outs = {}
    for name, bytes_ in (("aos", cache), ("soa", O.soa_from_aos(lay, cache))):
        lay_c = tq.layout_init(preset, G.D, name)
        tab = tq.Tables(lay_c, s)
        for dt in (torch.float16, torch.bfloat16, torch.float32):
            ko, vo = tq.dequant_kv(lay_c, torch.from_numpy(bytes_).cuda(), torch.from_numpy(table).cuda(), n,
                                   tab.signs, tab.centroids, out_dtype=dt)
            outs[(name, dt)] = (ko.cpu(), vo.cpu())
    for dt in (torch.float16, torch.bfloat16, torch.float32):
        assert torch.equal(outs[("aos", dt)][0], outs[("soa", dt)][0])
        assert torch.equal(outs[("aos", dt)][1], outs[("soa", dt)][1])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,S", [("llama8b", 8), ("longctx", 32), ("qwen32b", 8)])
def test_soa_full_size_matches_combined(name, S):
    """The decode workloads at full size, each stored by the GPU in both
    conventions from the same inputs: the SoA caches are the combined caches
    permuted (checked on sampled blocks) and the decode outputs are
    bit-identical (the combined decode is checked against the oracle at full
    size on sampled rows)."""
    import torch
    import quantized_decode_attention_tq_amd as tq
    import bench as B

    w = W.WORKLOADS[name]
    G.log(f"soa full size {name}")
    res = {}
    for bl in ("aos", "soa"):
        b = B.DecodeBench(torch, tq, w, S, block_layout=bl)
        b.stage1(0)
        b.stage2()
        torch.cuda.synchronize()
        res[bl] = (b.out.clone(), b.lse.clone(), b.caches[0])
        del b
    lay = O.layout(w.preset, G.D)
    rng = np.random.default_rng(0)
    for blk in rng.integers(0, res["aos"][2].shape[0], 8):
        a = res["aos"][2][int(blk)].cpu().numpy()[None]
        s = res["soa"][2][int(blk)].cpu().numpy()[None]
        np.testing.assert_array_equal(O.soa_from_aos(lay, a), s)
    assert torch.equal(res["aos"][0], res["soa"][0]) and torch.equal(res["aos"][1], res["soa"][1])
