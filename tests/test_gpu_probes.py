"""GPU checks of the hardware behaviour the kernels rely on, each with small,
in-bounds, single-wave probe launches: MFMA lane layouts, fp16 subnormal
operands through MFMA, the FP8 -> fp16 convert, and the device byte-permute
helpers against their host model."""

import numpy as np
import pytest

import oracle as O
import probe

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(7)


def _run_mfma(kind, a_lanes, b_lanes):
    import torch

    L = probe.lib()
    a = torch.from_numpy(np.ascontiguousarray(a_lanes).view(np.int32)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_lanes).view(np.int32)).cuda()
    d = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    f = L.tq_probe_mfma_16x16x32_f16 if kind == 32 else L.tq_probe_mfma_16x16x16_f16
    print(f"probe mfma 16x16x{kind}", flush=True)
    assert f(a.data_ptr(), b.data_ptr(), d.data_ptr()) == 0
    return d.cpu().numpy()


def _lanes(M, per):  # M: [16 rows/cols][K]; lane l holds row l%16, k = per*(l//16) + e
    out = np.zeros((64, per), np.float16)
    for l in range(64):
        out[l] = M[l % 16, per * (l // 16) : per * (l // 16) + per]
    return out.view(np.uint32)


@pytest.mark.parametrize("K", [32, 16])
def test_mfma_layout(K):
    per = K // 4
    A = RNG.integers(-8, 9, (16, K)).astype(np.float16)  # rows = M
    B = RNG.integers(-8, 9, (K, 16)).astype(np.float16)  # cols = N
    d = _run_mfma(K, _lanes(A, per), _lanes(B.T, per))
    C = A.astype(np.float64) @ B.astype(np.float64)
    for l in range(64):
        for r in range(4):
            assert d[l, r] == C[4 * (l // 16) + r, l % 16], (l, r)


def test_mfma_f16_subnormal_operands_are_exact():
    """Value codes enter the PV product as fp16 subnormals code * 2^(p-24)."""
    codes = RNG.integers(0, 16, (16, 16))
    pos = RNG.integers(0, 7, (16, 16))
    A = (codes * 2.0 ** (pos - 24)).astype(np.float16)
    assert np.all(A.astype(np.float64) == codes * 2.0 ** (pos - 24))
    B = RNG.integers(-60, 61, (16, 16)).astype(np.float16)  # sums stay exact in fp32
    d = _run_mfma(16, _lanes(A, 4), _lanes(B.T, 4))
    C = A.astype(np.float64) @ B.astype(np.float64)
    for l in range(64):
        for r in range(4):
            assert d[l, r] == np.float32(C[4 * (l // 16) + r, l % 16]), (l, r, d[l, r], C[4 * (l // 16) + r, l % 16])


def test_fp8_to_f16_convert_all_codes():
    import torch

    codes = np.arange(256, dtype=np.uint8)
    words = codes.view(np.uint32)  # 64 dwords, bytes 4i..4i+3
    din = torch.from_numpy(words.view(np.int32)).cuda()
    dout = torch.zeros(128, dtype=torch.int32, device="cuda")
    print("probe cvt fp8->f16", flush=True)
    assert probe.lib().tq_probe_cvt_fp8_f16(din.data_ptr(), dout.data_ptr(), 64) == 0
    halves = dout.cpu().numpy().view(np.uint16)  # order: bytes 0,1 then 2,3 of each dword
    got = halves.view(np.float16).astype(np.float64)
    want = O.fp8_e4m3fn_decode(codes)
    finite = np.isfinite(want)
    np.testing.assert_array_equal(got[finite], want[finite])
    assert np.all(np.isnan(got[~finite]))


@pytest.mark.parametrize("op", ["perm", "alignbyte", "key3_selectors", "lut8", "lut16", "val4_pairs", "val3_pairs",
                                "val2_pairs", "key2_selectors", "lm_value_selectors", "key3_pair_fields",
                                "key3_pair_entries", "key3_pair_windows", "lm4_value_selectors",
                                "lm2_value_selectors", "f32_to_e4m3"])
def test_device_bits_match_host_model(op):
    n = 4096
    inp = RNG.integers(0, 2 ** 32, (n, probe.N_IN), dtype=np.uint64).astype(np.uint32)
    if op == "perm":
        inp[:, 2] = RNG.integers(0, 16, (n, 4)).astype(np.uint32) @ np.array([1, 256, 65536, 2 ** 24], np.uint32)
    if op in ("lut8", "lut16"):
        inp[:, 0] &= 0x0F0F0F0F if op == "lut16" else 0x07070707
    if op == "f32_to_e4m3":
        x = np.concatenate([RNG.standard_normal(n // 2) * 100, RNG.standard_normal(n // 2) * 1e-3]).astype(np.float32)
        x[:4] = [np.inf, -np.inf, np.nan, -0.0]
        inp[:, 0] = x.view(np.uint32)
    print(f"probe bits {op}", flush=True)
    np.testing.assert_array_equal(probe.bits_device(op, inp), probe.bits_host(op, inp))


def test_permlane_swaps_pair_each_lane_with_its_partner():
    """The decode kernel's quarter reductions rely on permlane16_swap(v, v)
    leaving lane l holding {v[l], v[l ^ 16]} across its two results, and
    permlane32_swap(v, v) holding {v[l], v[l ^ 32]}; its Walsh-Hadamard
    butterflies on which result is which: the first holds the lane's own
    value where bit 4 (bit 5) of the lane is clear and the partner's where
    it is set, the second the other one."""
    import torch

    v = np.arange(64, dtype=np.uint32) * 7 + 1000
    din = torch.from_numpy(v.view(np.int32)).cuda()
    dout = torch.zeros(256, dtype=torch.int32, device="cuda")
    print("probe permlane swaps", flush=True)
    assert probe.lib().tq_probe_permlane_swap(din.data_ptr(), dout.data_ptr()) == 0
    out = dout.cpu().numpy().view(np.uint32).reshape(4, 64)
    for l in range(64):
        assert {int(out[0, l]), int(out[1, l])} == {int(v[l]), int(v[l ^ 16])}, l
        assert {int(out[2, l]), int(out[3, l])} == {int(v[l]), int(v[l ^ 32])}, l
        for row, bit in ((0, 16), (2, 32)):
            own, partner = int(v[l]), int(v[l ^ bit])
            first, second = (partner, own) if l & bit else (own, partner)
            assert (int(out[row, l]), int(out[row + 1, l])) == (first, second), (l, bit)


def test_wave_reductions_and_scan():
    """The decode's work search reduces and scans across the 64 lanes of a
    wave with DPP row operations and the row swaps: every lane gets the
    wave's sum and maximum, and lane l the sum of lanes 0..l."""
    import torch

    waves = 64
    x = RNG.integers(-(2 ** 20), 2 ** 20, (waves, 64)).astype(np.int32)
    x[0] = np.arange(64)  # a ramp
    x[1] = 0
    x[1, 63] = 5  # only the last lane
    x[2] = -7  # all equal, negative
    x[3] = RNG.integers(0, 1100, 64)  # work-search sized values
    din = torch.from_numpy(x.ravel()).cuda()
    dout = torch.zeros(192 * waves, dtype=torch.int32, device="cuda")
    print("probe wave ops", flush=True)
    assert probe.lib().tq_probe_wave_ops(din.data_ptr(), dout.data_ptr(), waves) == 0
    out = dout.cpu().numpy().reshape(waves, 3, 64).astype(np.int64)
    xs = x.astype(np.int64)
    np.testing.assert_array_equal(out[:, 0], np.repeat(xs.sum(1, keepdims=True), 64, 1))
    np.testing.assert_array_equal(out[:, 1], np.repeat(xs.max(1, keepdims=True), 64, 1))
    np.testing.assert_array_equal(out[:, 2], np.cumsum(xs, 1))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_hardware_fp8_encode_matches_software_encoder(kind):
    """The store kernel encodes FP8 keys with the hardware convert after
    clamping to [-448, 448] (NaN inputs take the software encoder): this pins
    that the hardware gives the software encoder's bytes (RNE) for every
    finite fp16 / bf16 input with |x| <= 448 -- above that it returns NaN
    where the encoder saturates, which the clamp covers."""
    import torch

    bits = np.arange(65536, dtype=np.uint32)
    x = O.widen(bits.astype(np.uint16), kind)
    f32 = x.astype(np.float32).view(np.uint32)
    din = torch.from_numpy(f32.view(np.int32)).cuda()
    dout = torch.zeros(3 * 65536, dtype=torch.int32, device="cuda")
    print(f"probe fp8 encode {kind}", flush=True)
    assert probe.lib().tq_probe_fp8_encode(din.data_ptr(), dout.data_ptr(), 65536) == 0
    out = dout.cpu().numpy().view(np.uint32).reshape(-1, 3)
    sw = out[:, 0]
    np.testing.assert_array_equal(sw, O.fp8_e4m3fn_encode(x))
    inr = np.isfinite(x) & (np.abs(x) <= 448)
    for col in (1, 2):
        np.testing.assert_array_equal(out[inr, col], sw[inr])


@pytest.mark.parametrize("block_size,row_bytes,groups", [(16, 1568, 7), (128, 944, 3), (32, 816, 40)])
def test_gather_read_covers_the_decode_tiles(block_size, row_bytes, groups):
    """The gather-read ceiling probe (the decode's tile reads without its
    arithmetic, timed by the benchmark) reads exactly the tiles of every
    sequence through the block table, split evenly over the workgroups: per
    workgroup, the XOR of its waves' outputs equals the XOR of every 32-bit
    word of its share of the tile list (an empty sequence included)."""
    import torch

    lens = np.array([1, 16, 0, 17, 250, 513, 64], np.int32)
    B = len(lens)
    bpseq = -(-lens // block_size)
    width = max(1, int(bpseq.max()))
    nb = int(bpseq.sum()) + 3
    perm = RNG.permutation(nb).astype(np.int32)
    table = np.zeros((B, width), np.int32)
    k = 0
    for b in range(B):
        table[b, : bpseq[b]] = perm[k : k + bpseq[b]]
        k += bpseq[b]
    tiles = -(-lens // 16)
    prefix = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)
    words = RNG.integers(0, 2 ** 32, nb * block_size * row_bytes // 4, dtype=np.uint64).astype(np.uint32)
    cache = torch.from_numpy(words.view(np.int32)).cuda()
    bt, pf = torch.from_numpy(table).cuda(), torch.from_numpy(prefix).cuda()
    out = torch.zeros(4 * groups, dtype=torch.int32, device="cuda")
    print(f"probe gather read bs={block_size} row={row_bytes} groups={groups}", flush=True)
    rc = probe.lib().tq_probe_gather_read(cache.data_ptr(), bt.data_ptr(), width, pf.data_ptr(), B, block_size,
                                          row_bytes, groups, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32).reshape(groups, 4), axis=1)
    rows = words.reshape(nb * block_size, row_bytes // 4)
    seq_of = np.repeat(np.arange(B), tiles)  # list tile -> sequence
    T = int(prefix[-1])
    for g in range(groups):
        want = np.uint32(0)
        for t in range(T * g // groups, T * (g + 1) // groups):
            b = seq_of[t]
            j = t - prefix[b]
            r0 = table[b, (j * 16) // block_size] * block_size + (j * 16) % block_size
            want ^= np.bitwise_xor.reduce(rows[r0 : r0 + 16].ravel())
        assert got[g] == want, g
