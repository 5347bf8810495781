"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (library routines, textbook tables, closed forms, invariants, brute
force, hand-derived bytes), chosen so that a plausible slip -- a dropped term,
a wrong sign or index, a transposed operand -- fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows


# ---------------------------------------------------------------- rotation


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy_sylvester(d):
    np.testing.assert_array_equal(O.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


def test_hadamard_matches_kronecker_recursion():
    h = np.array([[1.0]])
    for _ in range(7):
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    np.testing.assert_array_equal(O.hadamard(128), h)


def _fwht(x):
    """In-place butterfly (strides 1, 2, 4, ...), a different algorithm from
    the popcount definition."""
    y = np.array(x, dtype=np.float64)
    h = 1
    while h < y.shape[0]:
        for i in range(0, y.shape[0], 2 * h):
            a = y[i : i + h].copy()
            b = y[i + h : i + 2 * h].copy()
            y[i : i + h] = a + b
            y[i + h : i + 2 * h] = a - b
        h *= 2
    return y


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_properties(d):
    rng = np.random.default_rng(1)
    s = np.where(rng.integers(0, 2, d) == 1, -1.0, 1.0)
    R = O.rotation(s)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-12)
    x = rng.standard_normal(d)
    np.testing.assert_allclose(R.T @ (R @ x), x, atol=1e-12)
    # signs first, then the WHT: R x = FWHT(s * x) / sqrt(d)
    np.testing.assert_allclose(R @ x, _fwht(s * x) / math.sqrt(d), atol=1e-12)
    H = O.hadamard(d)
    np.testing.assert_array_equal(H @ H, d * np.eye(d))
    assert np.all(H[:, 0] == 1.0)
    # all-+1 signs reduce to the plain (unsigned, symmetric) Hadamard rotation
    np.testing.assert_allclose(O.rotation(np.ones(d)), scipy.linalg.hadamard(d) / math.sqrt(d), atol=0)
    # the signs act on the input side (columns), not the output side
    assert not np.allclose(R, (H * s[:, None]) / math.sqrt(d))


# ---------------------------------------------------------------- Lloyd-Max


def _quad_cell_mean(a, b, sigma):
    pdf = lambda x: math.exp(-0.5 * (x / sigma) ** 2) / (sigma * math.sqrt(2 * math.pi))
    num = scipy.integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    den = scipy.integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    return num / den


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_exact_fixed_point(bits):
    """Each centroid is the Gaussian conditional mean of its cell (computed
    here by adaptive quadrature, not the closed form) and each boundary is a
    midpoint."""
    d = 128
    sigma = 1.0 / math.sqrt(d)
    c, b = O.lloyd_max_exact(d, bits)
    assert c.shape == (1 << bits,) and b.shape == ((1 << bits) - 1,)
    np.testing.assert_allclose(b, (c[:-1] + c[1:]) / 2, atol=0)
    edges = [-12 * sigma] + list(b) + [12 * sigma]
    for i in range(len(c)):
        m = _quad_cell_mean(edges[i], edges[i + 1], sigma)
        assert abs(m - c[i]) < 1e-9 * sigma, (i, m, c[i])
    np.testing.assert_array_equal(c[::-1], -c)
    assert np.all(np.diff(c) > 0)


def test_lloyd_max_one_bit_closed_form():
    c, _ = O.lloyd_max_exact(128, 1)
    np.testing.assert_allclose(c, [-math.sqrt(2 / math.pi) / math.sqrt(128), math.sqrt(2 / math.pi) / math.sqrt(128)],
                               rtol=1e-13)


def test_lloyd_max_matches_max_1960_table():
    for levels, pos, mse in _read_table("gaussian_lloyd_max_max1960.txt"):
        levels = int(levels)
        bits = int(round(math.log2(levels)))
        want = np.array([float(v) for v in pos.split()])
        for d in (64, 128, 256):
            c, b = O.lloyd_max_exact(d, bits)
            got = c[levels // 2 :] * math.sqrt(d)
            # half a unit in the last of the table's 4 significant figures
            np.testing.assert_allclose(got, want, rtol=5e-4, atol=5e-5)
        # distortion of the quantizer, integrated numerically over every cell
        c, b = O.lloyd_max_exact(1, bits)
        edges = [-np.inf] + list(b) + [np.inf]
        pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
        dist = sum(scipy.integrate.quad(lambda x: (x - c[i]) ** 2 * pdf(x), edges[i], edges[i + 1])[0]
                   for i in range(levels))
        assert abs(dist - float(mse)) < 2e-4 * max(1.0, float(mse) * 100), (levels, dist, mse)


def test_codebook_tables_fp32_midpoints():
    for bits in (2, 3, 4):
        c32, b32 = O.codebook_tables(128, bits)
        assert c32.dtype == np.float32 and b32.dtype == np.float32
        np.testing.assert_array_equal(c32[::-1], -c32)
        np.testing.assert_array_equal(b32[::-1], -b32)
        # midpoint of two fp32 values: exact sum rounded once, then halved
        exact_mid = (c32[:-1].astype(np.float64) + c32[1:].astype(np.float64)) / 2
        np.testing.assert_array_equal(b32, exact_mid.astype(np.float32))
        assert b32[(1 << bits) // 2 - 1] == 0.0


def test_pages_trapz_solver_behaviour():
    """The pages' trapezoid solver converges at 3 bits and ends near the exact
    optimum (the trapezoid error on the +-10.5 sigma cells is ~1e-3 sigma)."""
    sigma = 1 / math.sqrt(128)
    for bits in (2, 3, 4):
        ct, bt = O.lloyd_max_pages_trapz(128, bits)
        ce, _ = O.lloyd_max_exact(128, bits)
        assert np.max(np.abs(ct - ce)) < 3e-3 * sigma
        assert np.max(np.abs(ct - ce)) > 1e-6 * sigma  # it is not the exact solver
        np.testing.assert_allclose(bt, (ct[:-1] + ct[1:]) / 2, atol=0)
    # with a fine trapezoid grid the same fixed-point iteration agrees with the
    # closed form; use the 3-bit case and check the trapezoid moments match quad
    c, b = O.lloyd_max_pages_trapz(128, 3)
    edges = [-10.5 * sigma] + list(b) + [10.5 * sigma]
    for i in range(8):
        m = _quad_cell_mean(edges[i], edges[i + 1], sigma)
        assert abs(m - c[i]) < 3e-3 * sigma


def _numpy_trapz_round(c, sigma):
    """One round of the pages' update (boundaries at midpoints, outer cells
    closed at +-10.5 sigma) with the cell moments from numpy's trapezoid rule
    over 201 equally spaced points per cell (200 intervals), vectorized."""
    edges = np.concatenate([[-10.5 * sigma], (c[:-1] + c[1:]) / 2, [10.5 * sigma]])
    x = np.linspace(edges[:-1], edges[1:], 201, axis=1)  # (cells, 201)
    pdf = np.exp(-x * x / (2 * sigma * sigma)) / math.sqrt(2 * math.pi * sigma * sigma)
    return np.trapezoid(x * pdf, x, axis=1) / np.trapezoid(pdf, x, axis=1)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pages_trapz_against_numpy_trapezoid(bits):
    """The pages' solver re-derived with numpy's trapezoid rule (a library
    routine) on the same 201-point cell grids: from the stated start (uniform
    over +-3.5 sigma), iterate until no centroid moves by 1e-10 -- returning
    the iterate from before that last update -- or for at most 200 rounds.
    The 2- and 3-bit runs stop on the tolerance; the 4-bit run hits the
    200-round cap, so its result depends on the start and on every round."""
    sigma = 1 / math.sqrt(128)
    L = 1 << bits
    c = -3.5 * sigma + 7.0 * sigma * (np.arange(L) + 0.5) / L
    rounds, converged = 0, False
    for _ in range(200):
        rounds += 1
        new = _numpy_trapz_round(c, sigma)
        if np.max(np.abs(new - c)) < 1e-10:
            converged = True
            break
        c = new
    info = {}
    got, gb = O.lloyd_max_pages_trapz(128, bits, info=info)
    assert info == {"rounds": rounds, "converged": converged}, (info, rounds, converged)
    assert converged == (bits < 4)
    np.testing.assert_allclose(got, c, rtol=0, atol=1e-13 * sigma)
    np.testing.assert_allclose(gb, (c[:-1] + c[1:]) / 2, rtol=0, atol=1e-13 * sigma)


def test_pages_trapz_start_and_cap():
    """Zero rounds return the stated start; the 4-bit iterate is still
    moving at the cap (one more round moves it by more than the tolerance)."""
    sigma = 1 / math.sqrt(128)
    c0, _ = O.lloyd_max_pages_trapz(128, 3, max_iter=0)
    np.testing.assert_allclose(c0, np.linspace(-3.5 * sigma, 3.5 * sigma, 9)[:-1] + 7 * sigma / 16, rtol=0,
                               atol=1e-15)
    c4, _ = O.lloyd_max_pages_trapz(128, 4)
    assert np.max(np.abs(_numpy_trapz_round(c4, sigma) - c4)) > 1e-10


# ---------------------------------------------------------------- signs


def test_splitmix64_reference_outputs():
    # Published first outputs of SplitMix64 seeded with 0 (the reference
    # generator used to seed xoshiro/xoroshiro).
    assert O.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_wht_signs_deterministic_and_balanced():
    s = O.wht_signs(128, 42)
    np.testing.assert_array_equal(s, O.wht_signs(128, 42))
    assert set(np.unique(s)) <= {-1.0, 1.0}
    assert not np.array_equal(s, O.wht_signs(128, 43))
    big = O.wht_signs(20000, 7)
    assert abs(big.mean()) < 0.03
    assert s[0] == -1.0  # top bit of 0x... first draw for seed 42, recomputed below
    z = O.splitmix64(42, 1)[0]
    assert (z >> 63) == 1


# ---------------------------------------------------------------- number formats


def test_fp8_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.fp8_e4m3fn_decode(codes)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_encode_every_16bit_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = O.widen(bits, dtype)
    finite = np.isfinite(x)
    inrange = finite & (np.abs(x) <= 448.0)
    got = O.fp8_e4m3fn_encode(x)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    want = torch.from_numpy(bits.view(np.int16)).view(tdt)[torch.from_numpy(inrange)]
    want = want.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got[inrange], want)
    # beyond the range: saturate to +-448 (0x7E / 0xFE)
    big = finite & (np.abs(x) > 448.0)
    assert np.all((got[big] & 0x7F) == 0x7E)
    np.testing.assert_array_equal(got[big] >> 7, (x[big] < 0).astype(np.uint8))
    # round trip of every finite e4m3 value
    vals = O.fp8_e4m3fn_decode(np.arange(256))
    ok = np.isfinite(vals)
    np.testing.assert_array_equal(O.fp8_e4m3fn_encode(vals[ok]), np.arange(256)[ok].astype(np.uint8) & np.where(vals[ok] == 0, 0xFF, 0xFF))


def test_fp16_field_encoding():
    assert O.fp16_bits(1.0) == 0x3C00
    assert O.fp16_bits(65504.0) == 0x7BFF
    assert O.fp16_bits(2.0 ** -24) == 0x0001
    assert O.fp16_bits(1.0 + 2.0 ** -11) == 0x3C00  # tie -> even
    assert O.fp16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02  # tie -> even (up)


def test_widen_bf16_exact():
    assert O.widen(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert O.widen(np.array([0xC0A0], np.uint16), "bf16")[0] == -5.0
    b = W.to_bits(np.array([1.0 + 2.0 ** -8], np.float32), "bf16")  # tie -> even
    assert b[0] == 0x3F80


# ---------------------------------------------------------------- packing


def test_pack_hand_examples():
    for bits, codes, want in _read_table("pack_examples.txt"):
        bits = int(bits)
        codes = np.array([int(c) for c in codes.split()])
        want = bytes(int(h, 16) for h in want.split())
        got = O.pack_lsb(codes, bits).tobytes()
        assert got == want, (bits, codes, got.hex(), want.hex())
        np.testing.assert_array_equal(O.unpack_lsb(np.frombuffer(want, np.uint8), bits, len(codes)), codes)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip_exhaustive(bits):
    L = 1 << bits
    rng = np.random.default_rng(bits)
    # every code value at every position of a 128-code vector (one row per
    # (value, position), the other positions random)
    codes = rng.integers(0, L, (L * 128, 128))
    v, pos = np.divmod(np.arange(L * 128), 128)
    codes[np.arange(L * 128), pos] = v
    packed = O.pack_lsb(codes, bits)
    assert packed.shape == (L * 128, 128 * bits // 8)
    np.testing.assert_array_equal(O.unpack_lsb(packed, bits, 128), codes)
    codes = rng.integers(0, L, (500, 128))
    np.testing.assert_array_equal(O.unpack_lsb(O.pack_lsb(codes, bits), bits, 128), codes)


def test_layout_sizes():
    want = {"turboquant_k8v4": (128, 128, 64, 68, 196), "turboquant_4bit_nc": (64, 66, 64, 68, 134),
            "turboquant_k3v4_nc": (48, 50, 64, 68, 118), "turboquant_3bit_nc": (48, 50, 48, 52, 102),
            "turboquant_k8v3": (128, 128, 48, 52, 180), "turboquant_k4v3_nc": (64, 66, 48, 52, 118),
            "turboquant_2bit_nc": (32, 34, 32, 36, 70), "turboquant_k8v3lm": (128, 128, 48, 50, 178),
            "turboquant_3bit_lm": (48, 50, 48, 50, 100)}
    for p, (kd, kps, vd, vps, slot) in want.items():
        L = O.layout(p, 128)
        assert (L.key_data_bytes, L.key_packed_size, L.value_data_bytes, L.value_packed_size, L.slot_size_aligned) == \
            (kd, kps, vd, vps, slot)
    # "2.6x" KV compression for k8v4 against 16-bit K+V
    assert round(2 * 128 * 2 / O.layout("turboquant_k8v4", 128).slot_size_aligned, 1) == 2.6
    assert O.layout("turboquant_3bit_nc", 100).slot_size_aligned % 2 == 0
    assert O.kv_cache_shape(O.layout("turboquant_3bit_nc", 128), 10, 16, 8) == (10, 16, 8, 102)


# ---------------------------------------------------------------- quantizers


def test_bucketize_ties_and_ends():
    b = np.array([-1.0, 0.0, 1.0], dtype=np.float32)
    u = np.array([-2.0, -1.0, -0.5, 0.0, -0.0, 0.5, 1.0, 2.0])
    np.testing.assert_array_equal(O.bucketize(u, b), [0, 0, 1, 1, 1, 2, 2, 3])
    np.testing.assert_array_equal(O.bucketize(u, b), torch.bucketize(torch.tensor(u), torch.tensor(b, dtype=torch.float64), right=False).numpy())


@pytest.mark.parametrize("bits,distortion", [(2, 0.1175), (3, 0.03455), (4, 0.009497)])
@pytest.mark.parametrize("d", [128, 256])
def test_mse_key_reconstruction_statistics(bits, distortion, d):
    """Gaussian keys: relative squared error of gamma R^T c[code] is close to
    the Lloyd-Max distortion, and the norm correction matches norms."""
    rng = np.random.default_rng(bits)
    c32, b32 = O.codebook_tables(d, bits)
    s = np.where(rng.integers(0, 2, d) == 1, -1.0, 1.0)
    R = O.rotation(s)
    errs = []
    for _ in range(300):
        x = rng.standard_normal(d) * rng.uniform(0.1, 10)
        codes, gamma = O.quantize_key_mse(x, R, c32, b32, True)
        chat = c32[codes].astype(np.float64)
        xr = gamma * (R.T @ chat)
        assert abs(np.linalg.norm(xr) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)
        errs.append(np.sum((xr - x) ** 2) / np.sum(x ** 2))
    rel = float(np.mean(errs))
    assert 0.8 * distortion < rel < 1.25 * distortion, rel
    # E||c[code]||^2 ~ 1 - distortion for unit-norm inputs (no correction)
    norms = []
    for _ in range(300):
        x = rng.standard_normal(d)
        codes, _ = O.quantize_key_mse(x, R, c32, b32, False)
        norms.append(np.sum(c32[codes].astype(np.float64) ** 2))
    assert abs(np.mean(norms) - (1 - distortion)) < 0.25 * distortion


def test_mse_key_zero_vector():
    c32, b32 = O.codebook_tables(D, 4)
    codes, gamma = O.quantize_key_mse(np.zeros(D), O.rotation(np.ones(D)), c32, b32, True)
    assert gamma == 0.0 and np.all(codes == 7)


def test_value_codec_properties():
    rng = np.random.default_rng(5)
    for bits in (3, 4):
        L = (1 << bits) - 1
        for _ in range(200):
            v = O.widen(W.to_bits(rng.standard_normal(D) * rng.uniform(0.01, 20), "bf16"), "bf16")
            codes, s16, z16 = O.quantize_values(v, bits)
            s = float(np.uint16(s16).view(np.float16))
            z = float(np.uint16(z16).view(np.float16))
            assert codes.min() >= 0 and codes.max() <= L
            vhat = z + s * codes
            # half a step, plus the fp16 rounding of zero and of the scale over L steps
            bound = s / 2 + abs(z) * 2 ** -11 + L * s * 2 ** -11 + 1e-12
            assert np.max(np.abs(vhat - v)) <= bound * 1.0001
    # hand example: 0, 0.5, ..., 7.5 at 4 bits -> zero 0, scale 0.5, codes 0..15
    v = np.arange(16) * 0.5
    codes, s16, z16 = O.quantize_values(np.tile(v, 8), 4)
    assert s16 == 0x3800 and z16 == 0x0000
    np.testing.assert_array_equal(codes, np.tile(np.arange(16), 8))
    # constant vector: scale 0, all codes 0, reconstruction exact
    codes, s16, z16 = O.quantize_values(np.full(D, 3.25), 4)
    assert s16 == 0 and np.all(codes == 0) and float(np.uint16(z16).view(np.float16)) == 3.25


def _fp16_nearest_even(q):
    """Exact rational q -> the nearest binary16 value (ties to the even
    significand), by comparing q with the representable neighbours."""
    from fractions import Fraction

    f = np.float16(float(q))  # within one step of the answer
    cands = sorted({np.nextafter(f, np.float16(-np.inf)), f, np.nextafter(f, np.float16(np.inf))},
                   key=lambda h: (abs(Fraction(float(h)) - q), int(np.array(h).view(np.uint16)) & 1))
    return cands[0]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_codes_exact_definition(bits):
    """Value fields and codes equal the definition evaluated in rational
    arithmetic: zero = fp16(min v), scale = fp16((max - min) / (2^b - 1))
    (round to nearest even), code = clamp(floor((v - z) / s + 1/2)); ties
    round up."""
    from fractions import Fraction

    levels = (1 << bits) - 1
    rng = np.random.default_rng(40 + bits)
    for r in range(60):
        v = O.widen(W.to_bits(rng.standard_normal(D) * rng.uniform(0.001, 50) + rng.uniform(-3, 3), "bf16"), "bf16")
        codes, s16, z16 = O.quantize_values(v, bits)
        z = np.uint16(z16).view(np.float16)
        s = np.uint16(s16).view(np.float16)
        assert z == _fp16_nearest_even(Fraction(float(v.min())))
        assert s == _fp16_nearest_even((Fraction(float(v.max())) - Fraction(float(v.min()))) / levels)
        zf, sf = Fraction(float(z)), Fraction(float(s))
        for i in range(D):
            x = (Fraction(float(v[i])) - zf) / sf + Fraction(1, 2)
            want = min(max(x.numerator // x.denominator, 0), levels)
            assert codes[i] == want, (r, i, codes[i], want)
    # exact ties: v - z = (k + 1/2) s rounds up to k + 1; just below stays at k
    z, s = 0.25, 0.1875  # fp16 values; (k + 1/2) * 0.1875 is exact in float64
    k = np.arange(levels)
    ties = z + (k + 0.5) * s
    vt = np.concatenate([[z], ties, np.nextafter(ties, -np.inf)])
    got = O.value_codes(vt[None, :], np.array([z]), np.array([s]), bits)[0]
    np.testing.assert_array_equal(got[1 : 1 + levels], k + 1)
    np.testing.assert_array_equal(got[1 + levels :], k)
    assert got[0] == 0


def test_workspace_bytes_of_the_pages_layout():
    """(B, Hq, S, D+1) fp32: 2 641 920 bytes for 4 sequences, 40 query heads,
    32 splits, head_dim 128 (the long-context decode shape)."""
    assert O.workspace_bytes(4, 40, 128, 32) == 2641920
    assert O.workspace_bytes(32, 32, 128, 8) == 32 * 32 * 8 * 129 * 4


def test_encode_decode_slot_roundtrip():
    rng = np.random.default_rng(9)
    for preset in O.PRESETS:
        lay = O.layout(preset, D)
        s = np.where(rng.integers(0, 2, D) == 1, -1.0, 1.0)
        R = O.rotation(s)
        c32, b32 = (None, None) if lay.key_fp8 else O.codebook_tables(D, lay.key_bits)
        k = O.widen(W.to_bits(rng.standard_normal(D) * 2, "bf16"), "bf16")
        v = O.widen(W.to_bits(rng.standard_normal(D), "bf16"), "bf16")
        slot = O.encode_slot(lay, k, v, R, c32, b32)
        assert slot.shape == (lay.slot_size_aligned,)
        kh, vh = O.decode_slot(lay, slot, c32, R)
        if lay.key_fp8:
            np.testing.assert_array_equal(slot[:D], O.fp8_e4m3fn_encode(k))
            assert np.max(np.abs(kh - k)) <= np.max(np.abs(k)) * 2 ** -4
        else:
            # rotated domain: back-rotate and compare with the input
            kr = R.T @ kh
            assert np.linalg.norm(kr - k) / np.linalg.norm(k) < {2: 0.45, 3: 0.3}.get(lay.key_bits, 0.2)
            np.testing.assert_allclose(np.linalg.norm(kh), np.linalg.norm(k), rtol=1e-3)
        if lay.value_lm:  # original space already; the matched norm keeps ||v||
            # Lloyd-Max distortion of N(0, 1) at 2 / 3 / 4 bits: 0.118 / 0.035 / 0.0095
            assert np.linalg.norm(vh - v) / np.linalg.norm(v) < {2: 0.45, 3: 0.3}.get(lay.value_bits, 0.2)
            np.testing.assert_allclose(np.linalg.norm(vh), np.linalg.norm(v), rtol=1e-3)
        else:
            assert np.max(np.abs(vh - v)) < (np.max(v) - np.min(v)) / ((1 << lay.value_bits) - 1)


# ---------------------------------------------------------------- decode


def _tiny_cache(preset, B=2, Hq=4, Hk=2, bs=16, lens=(37, 5), seed=0, dtype="bf16"):
    rng = np.random.default_rng(seed)
    lay = O.layout(preset, D)
    s = np.where(rng.integers(0, 2, D) == 1, -1.0, 1.0)
    c32, b32 = (None, None) if lay.key_fp8 else O.codebook_tables(D, lay.key_bits)
    nbl = [-(-L // bs) for L in lens]
    nb = sum(nbl) + 3
    perm = rng.permutation(nb)
    table = np.full((B, max(nbl)), -1, dtype=np.int64)
    pos = 0
    for b in range(B):
        table[b, : nbl[b]] = perm[pos : pos + nbl[b]]
        pos += nbl[b]
    cache = np.zeros((nb, bs, Hk, lay.slot_size_aligned), dtype=np.uint8)
    K = [O.widen(W.to_bits(rng.standard_normal((L, Hk, D)), dtype), dtype) for L in lens]
    V = [O.widen(W.to_bits(rng.standard_normal((L, Hk, D)), dtype), dtype) for L in lens]
    for b, L in enumerate(lens):
        slots = table[b, np.arange(L) // bs] * bs + np.arange(L) % bs
        O.store(lay, K[b], V[b], slots, cache, s, c32, b32)
    q = O.widen(W.to_bits(rng.standard_normal((B, Hq, D)), dtype), dtype)
    return lay, s, c32, table, np.array(lens), cache, q, K, V


@pytest.mark.parametrize("preset", list(O.PRESETS))
def test_decode_matches_sdpa_on_dequantized_cache(preset):
    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache(preset)
    scale = 1 / math.sqrt(D)
    out, lse = O.decode(lay, q, cache, table, lens, s, c32, scale)
    B, Hq, _ = q.shape
    g = Hq // cache.shape[2]
    for b in range(B):
        for hq in range(Hq):
            Kd, Vd = O.dequant_original_space(lay, cache, table[b], int(lens[b]), hq // g, s, c32)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(q[b, hq])[None, None, None], torch.tensor(Kd)[None, None], torch.tensor(Vd)[None, None],
                scale=scale)[0, 0, 0].numpy()
            np.testing.assert_allclose(out[b, hq], ref, rtol=1e-10, atol=1e-12)
            sc = scale * Kd @ q[b, hq]
            assert abs(lse[b, hq] - (sc.max() + math.log(np.exp(sc - sc.max()).sum()))) < 1e-10


def test_decode_close_to_unquantized_attention():
    """End to end (store then decode) against attention on the raw K/V.  Each
    query points at one stored key, so the softmax is peaked and a wrong
    rotation, sign, norm or gather index moves the output far; the honest
    error is the quantization error of the few dominant rows."""
    rng = np.random.default_rng(11)
    for preset, tol in (("turboquant_4bit_nc", 0.08), ("turboquant_k8v4", 0.08), ("turboquant_k3v4_nc", 0.12),
                        ("turboquant_3bit_nc", 0.2)):
        lay, s, c32, table, lens, cache, q, K, V = _tiny_cache(preset, lens=(200, 64))
        scale = 1 / math.sqrt(D)
        g = q.shape[1] // cache.shape[2]
        for b in range(q.shape[0]):
            for hq in range(q.shape[1]):
                # first token, last token, then random ones: an off-by-one
                # gather window misses the ends
                tgt = [0, lens[b] - 1][hq] if hq < 2 else rng.integers(0, lens[b])
                kt = K[b][tgt, hq // g]
                q[b, hq] = kt * (12.0 / (scale * np.dot(kt, kt)))
        out, _ = O.decode(lay, q, cache, table, lens, s, c32, scale)
        for b in range(q.shape[0]):
            for hq in range(q.shape[1]):
                ref, _ = O.attend(q[b, hq], K[b][:, hq // g], V[b][:, hq // g], scale)
                err = np.max(np.abs(out[b, hq] - ref)) / np.max(np.abs(ref))
                assert err < tol, (preset, b, hq, err)


def test_decode_special_cases():
    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache("turboquant_4bit_nc", lens=(1, 0))
    out, lse = O.decode(lay, q, cache, table, lens, s, c32, 0.1)
    _, Vd = O.dequant_original_space(lay, cache, table[0], 1, 0, s, c32)
    np.testing.assert_allclose(out[0, 0], Vd[0], rtol=0, atol=0)  # L = 1 -> o = v
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))  # L = 0 -> 0, -inf
    # equal scores (zero query) -> mean of the values
    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache("turboquant_k8v4", lens=(21, 3))
    q[:] = 0.0
    out, _ = O.decode(lay, q, cache, table, lens, s, c32, 0.1)
    _, Vd = O.dequant_original_space(lay, cache, table[0], 21, 0, s, c32)
    np.testing.assert_allclose(out[0, 0], Vd.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_decode_gqa_one_reduces_to_mha():
    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache("turboquant_3bit_nc", Hq=2, Hk=2)
    out, _ = O.decode(lay, q, cache, table, lens, s, c32, 0.1)
    for h in range(2):
        Kd, Vd = O.gather_sequence(lay, cache, table[0], int(lens[0]), h, c32)
        o, _ = O.attend(O.rotation(s) @ q[0, h], Kd, Vd, 0.1)
        np.testing.assert_allclose(out[0, h], o, rtol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 32, 100])
def test_split_merge_equals_unsplit(S):
    rng = np.random.default_rng(S)
    K = rng.standard_normal((300, D))
    V = rng.standard_normal((300, D))
    q = rng.standard_normal(D) * 2
    o1, l1 = O.attend(q, K, V, 0.2)
    o2, l2 = O.decode_split(q, K, V, 0.2, S, 16)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    assert abs(l2 - l1) < 1e-12
    rng_parts = O.split_ranges(300, S, 16)
    assert rng_parts[0][0] == 0 and rng_parts[-1][1] == 300
    assert all(a % 16 == 0 for a, _ in rng_parts if a < 300)


def test_store_skips_negative_slots_and_touches_nothing_else():
    lay = O.layout("turboquant_k3v4_nc", D)
    c32, b32 = O.codebook_tables(D, 3)
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 256, (4, 16, 2, lay.slot_size_aligned)).astype(np.uint8)
    before = cache.copy()
    k = rng.standard_normal((3, 2, D))
    O.store(lay, k, k, np.array([5, -1, 40]), cache, np.ones(D), c32, b32)
    changed = np.argwhere(np.any(cache != before, axis=-1))
    assert {tuple(x) for x in changed} <= {(0, 5, 0), (0, 5, 1), (2, 8, 0), (2, 8, 1)}


def test_block_table_indirection():
    """Same tokens stored under a permuted table decode identically."""
    lay = O.layout("turboquant_4bit_nc", D)
    c32, b32 = O.codebook_tables(D, 4)
    rng = np.random.default_rng(4)
    L, bs = 70, 16
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 2, D))
    outs = []
    for table in (np.arange(5), np.array([4, 0, 3, 1, 2])):
        cache = np.zeros((5, bs, 1, lay.slot_size_aligned), np.uint8)
        O.store(lay, k, v, table[np.arange(L) // bs] * bs + np.arange(L) % bs, cache, np.ones(D), c32, b32)
        outs.append(O.decode(lay, q, cache, table[None], np.array([L]), np.ones(D), c32, 0.1)[0])
    np.testing.assert_array_equal(outs[0], outs[1])


@pytest.mark.parametrize("preset", list(O.PRESETS))
def test_row_vectorized_store_equals_per_row_store(preset):
    lay = O.layout(preset, D)
    rng = np.random.default_rng(21)
    c32, b32 = (None, None) if lay.key_fp8 else O.codebook_tables(D, lay.key_bits)
    s = np.where(rng.integers(0, 2, D) == 1, -1.0, 1.0)
    N, Hk, bs = 40, 3, 16
    k = O.widen(W.to_bits(rng.standard_normal((N, Hk, D)) * rng.uniform(0.1, 8, (1, Hk, D)), "bf16"), "bf16")
    v = O.widen(W.to_bits(rng.standard_normal((N, Hk, D)) * 3, "bf16"), "bf16")
    k[3, 1] = 0.0  # zero key
    v[5, 2] = 1.5  # constant value row
    slots = rng.permutation(4 * bs)[:N]
    slots[7] = -1
    c1 = np.zeros((4, bs, Hk, lay.slot_size_aligned), np.uint8)
    c2 = c1.copy()
    O.store(lay, k, v, slots, c1, s, c32, b32)
    O.store_rows(lay, k, v, slots, c2, s, c32, b32)
    np.testing.assert_array_equal(c1, c2)


@pytest.mark.parametrize("preset", list(O.PRESETS))
def test_row_vectorized_decode_equals_per_slot_decode(preset):
    lay = O.layout(preset, D)
    rng = np.random.default_rng(22)
    c32, b32 = (None, None) if lay.key_fp8 else O.codebook_tables(D, lay.key_bits)
    R = O.rotation(np.where(rng.integers(0, 2, D) == 1, -1.0, 1.0))
    k = O.widen(W.to_bits(rng.standard_normal((30, D)) * 2, "bf16"), "bf16")
    v = O.widen(W.to_bits(rng.standard_normal((30, D)), "bf16"), "bf16")
    slots = O.encode_slots(lay, k, v, R, c32, b32)
    K, V = O.decode_slots(lay, slots, c32, R)
    for i in range(30):
        ki, vi = O.decode_slot(lay, slots[i], c32, R)
        np.testing.assert_array_equal(K[i], ki)
        if lay.value_lm:  # a matrix and a vector product: the sums may round apart
            np.testing.assert_allclose(V[i], vi, rtol=1e-13, atol=1e-15)
        else:
            np.testing.assert_array_equal(V[i], vi)


# ------------------------------------------------------- dequant (original space)
# Mean squared error of the Lloyd-Max quantizer for a unit Gaussian, from
# J. Max, "Quantizing for minimum distortion" (1960), table of optimum
# quantizers: N = 8 and N = 16 levels.
MAX_GAUSSIAN_DISTORTION = {2: 0.1175, 3: 0.03454, 4: 0.009497}


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc",
                                    "turboquant_k4v3_nc", "turboquant_2bit_nc", "turboquant_3bit_lm",
                                    "turboquant_k8v3lm"])
@pytest.mark.parametrize("d", [128, 256])
def test_dequant_original_space_error_matches_lloyd_max_distortion(preset, d):
    """Store then dequantize back to the original space: after the randomized
    Hadamard rotation the coordinates are near-Gaussian ([TQ+] "Background":
    why the sign vector matters), so the relative key error averages out at
    the Gaussian Lloyd-Max distortion of the key bit width.  Applying the
    rotation instead of its transpose, or dropping the signs, gives about 2.
    Values: the uniform quantizer's error bound (half a step plus the zero
    point's fp16 rounding)."""
    rng = np.random.default_rng(5)
    lay = O.layout(preset, d)
    c32, b32 = O.codebook_tables(d, lay.key_bits)
    s = O.wht_signs(d, 3)
    N, bs = 400, 16
    K = O.widen(W.to_bits(rng.standard_normal((N, 1, d)) * np.exp(0.3 * rng.standard_normal((1, 1, d))), "bf16"),
                "bf16")
    V = O.widen(W.to_bits(rng.standard_normal((N, 1, d)), "bf16"), "bf16")
    cache = np.zeros((N // bs, bs, 1, lay.slot_size_aligned), np.uint8)
    O.store_rows(lay, K, V, np.arange(N), cache, s, c32, b32)
    Kd, Vd = O.dequant_original_space(lay, cache, np.arange(N // bs), N, 0, s, c32)
    k, v = K[:, 0], V[:, 0]
    if not lay.key_fp8:
        rel = np.sum((k - Kd) ** 2, axis=1) / np.sum(k ** 2, axis=1)
        ratio = rel.mean() / MAX_GAUSSIAN_DISTORTION[lay.key_bits]
        assert 0.85 < ratio < 1.1, ratio
    if lay.value_lm:  # values take the same rotation and codebook: the same distortion
        rel = np.sum((v - Vd) ** 2, axis=1) / np.sum(v ** 2, axis=1)
        ratio = rel.mean() / MAX_GAUSSIAN_DISTORTION[lay.value_bits]
        assert 0.85 < ratio < 1.1, ratio
        return
    levels = (1 << lay.value_bits) - 1
    step = np.float16((v.max(1) - v.min(1)).astype(np.float32) / np.float32(levels)).astype(np.float64)
    zerr = np.abs(np.float16(v.min(1)).astype(np.float64) - v.min(1))
    assert np.all(np.abs(v - Vd) <= (0.5 * step + zerr)[:, None] * (1 + 1e-6) + 1e-12)


def test_dequant_original_space_fp8_keys_are_the_e4m3_values():
    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache("turboquant_k8v4", lens=(37, 5))
    for b, L in enumerate(lens):
        for h in range(cache.shape[2]):
            Kd, _ = O.dequant_original_space(lay, cache, table[b], int(L), h, s, c32)
            want = O.fp8_e4m3fn_decode(O.fp8_e4m3fn_encode(K[b][:, h]))
            np.testing.assert_array_equal(Kd, want)


# ---------------------------------------------------------------- SoA layout

# Per preset at head_dim 128: (data bytes per row = key data + value data,
# u16 metadata fields per row), the constants of the pages' SoA reader ([API]
# _continuation_prefill: data bytes per slot, NUM_SOA_FIELDS 2 for FP8 keys
# and 3 otherwise).
SOA_CONSTANTS = {
    "turboquant_k8v4": (128 + 64, 2),
    "turboquant_4bit_nc": (64 + 64, 3),
    "turboquant_k3v4_nc": (48 + 64, 3),
    "turboquant_3bit_nc": (48 + 48, 3),
    "turboquant_k8v3": (128 + 48, 2),
    "turboquant_k4v3_nc": (64 + 48, 3),
    "turboquant_2bit_nc": (32 + 32, 3),
    "turboquant_k8v3lm": (128 + 48, 1),
    "turboquant_3bit_lm": (48 + 48, 2),
    "turboquant_k8v4lm": (128 + 64, 1),
    "turboquant_4bit_lm": (64 + 64, 2),
    "turboquant_2bit_lm": (32 + 32, 2),
}


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("bs,Hk", [(16, 1), (16, 8), (64, 3), (128, 2)])
def test_soa_geometry_matches_the_pages_constants(preset, bs, Hk):
    """Metadata region offset = block_size * Hk * data bytes per slot, and the
    two regions fill exactly the combined cache's block (same tensor shape,
    [API] _store_kv)."""
    lay = O.layout(preset, D)
    data, meta, nf = O.soa_geometry(lay, bs, Hk)
    assert (data, nf) == SOA_CONSTANTS[preset]
    assert meta == bs * Hk * data
    assert meta + bs * Hk * 2 * nf == bs * Hk * lay.slot_size_aligned


@pytest.mark.parametrize("preset", O.PRESETS)
def test_soa_conversion_is_a_byte_permutation(preset):
    """Every byte of a block lands in exactly one place and comes back: with
    all slot bytes distinct (as 16-bit tags carried in two byte planes) the
    SoA block holds each tag once, and the inverse restores the cache."""
    lay = O.layout(preset, D)
    bs, Hk, slot = 16, 3, lay.slot_size_aligned
    n = bs * Hk * slot
    tags = np.arange(n, dtype=np.int64).reshape(1, bs, Hk, slot)
    lo = O.soa_from_aos(lay, (tags & 0xFF).astype(np.uint8)).astype(np.int64)
    hi = O.soa_from_aos(lay, (tags >> 8).astype(np.uint8)).astype(np.int64)
    assert sorted((lo | (hi << 8)).ravel().tolist()) == list(range(n))
    rng = np.random.default_rng(1)
    c = rng.integers(0, 256, (4, bs, Hk, slot), dtype=np.uint8)
    np.testing.assert_array_equal(O.aos_from_soa(lay, O.soa_from_aos(lay, c)), c)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_k3v4_nc"])
def test_soa_field_positions_of_one_slot(preset):
    """Hand-placed example: the slot of token 3, KV head 1 in a block of 16
    tokens x 2 heads is row r = 3 * 2 + 1 = 7.  Its key data and value data
    follow each other at 7 * data; its norm (MSE keys), scale and zero are the
    u16 fields 0..2 (FP8: scale, zero = 0, 1) of row 7 in the metadata
    region."""
    lay = O.layout(preset, D)
    bs, Hk = 16, 2
    data, meta, nf = O.soa_geometry(lay, bs, Hk)
    cache = np.zeros((1, bs, Hk, lay.slot_size_aligned), np.uint8)
    s = cache[0, 3, 1]
    kd, vd, kps = lay.key_data_bytes, lay.value_data_bytes, lay.key_packed_size
    s[:kd] = 0x11
    s[kps : kps + vd] = 0x33
    if not lay.key_fp8:
        s[kd : kd + 2] = [0xA1, 0xA2]
    s[kps + vd : kps + vd + 4] = [0xB1, 0xB2, 0xC1, 0xC2]
    flat = O.soa_from_aos(lay, cache).reshape(-1)
    want = np.zeros_like(flat)
    want[7 * data : 7 * data + kd] = 0x11
    want[7 * data + kd : 8 * data] = 0x33
    fields = ([[0xA1, 0xA2]] if not lay.key_fp8 else []) + [[0xB1, 0xB2], [0xC1, 0xC2]]
    for f, v in enumerate(fields):
        want[meta + 2 * (7 * nf + f) : meta + 2 * (7 * nf + f) + 2] = v
    np.testing.assert_array_equal(flat, want)


def test_soa_store_equals_converted_combined_store():
    """Storing into an SoA cache that already holds rows leaves the other
    rows untouched and writes the new ones as the combined store would."""
    rng = np.random.default_rng(2)
    lay = O.layout("turboquant_3bit_nc", D)
    c32, b32 = O.codebook_tables(D, 3)
    s = O.wht_signs(D, 1)
    bs, Hk, nb = 32, 2, 3
    K = rng.standard_normal((40, Hk, D))
    V = rng.standard_normal((40, Hk, D))
    slots = rng.permutation(nb * bs)[:40]
    aos = np.zeros((nb, bs, Hk, lay.slot_size_aligned), np.uint8)
    O.store_rows(lay, K[:25], V[:25], slots[:25], aos, s, c32, b32)
    soa = O.soa_from_aos(lay, aos)
    O.store_rows(lay, K[25:], V[25:], slots[25:], aos, s, c32, b32)
    O.store_soa(lay, K[25:], V[25:], slots[25:], soa, s, c32, b32)
    np.testing.assert_array_equal(soa, O.soa_from_aos(lay, aos))


# ---------------------------------------------------------------- sinks and sliding window


def _qkv(n, seed=0, D=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))


def test_sink_closed_form_against_no_sink():
    """A sink logit only adds e^sink to the denominator: o_sink = o * e^lse /
    (e^lse + e^sink) and lse_sink = logaddexp(lse, sink), for sinks below,
    near and above the scores."""
    q, K, V = _qkv(23, 1)
    o0, l0 = O.attend(q, K, V, 0.3)
    for sink in (-30.0, -1.0, 0.0, l0, 2.5, 40.0):
        o, l = O.attend(q, K, V, 0.3, sink)
        np.testing.assert_allclose(l, np.logaddexp(l0, sink), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o, o0 * math.exp(l0 - np.logaddexp(l0, sink)), rtol=1e-11, atol=1e-14)
    o, l = O.attend(q, K, V, 0.3, -math.inf)
    np.testing.assert_array_equal(o, o0)
    assert l == l0


def test_sink_is_a_zero_valued_extra_logit():
    """Brute force with a library softmax: scores plus the sink, values plus a
    zero row."""
    import scipy.special

    q, K, V = _qkv(9, 2)
    sink = 0.7
    w = scipy.special.softmax(np.append(0.5 * (K @ q), sink))
    o, l = O.attend(q, K, V, 0.5, sink)
    np.testing.assert_allclose(o, w[:-1] @ V, rtol=1e-12)
    np.testing.assert_allclose(l, scipy.special.logsumexp(np.append(0.5 * (K @ q), sink)), rtol=1e-13)
    # no tokens: the output is 0 and the LSE is the sink alone
    o, l = O.attend(q, K[:0], V[:0], 0.5, sink)
    assert np.all(o == 0) and l == sink


def test_sink_survives_the_split_merge():
    q, K, V = _qkv(100, 3)
    want = O.attend(q, K, V, 0.2, 1.3)
    for S in (1, 3, 8):
        o, l = O.decode_split(q, K, V, 0.2, S, 16, 1.3)
        np.testing.assert_allclose(o, want[0], rtol=1e-11)
        np.testing.assert_allclose(l, want[1], rtol=1e-12)


def test_sliding_window_closed_forms():
    """Window 1: the softmax over one token is that token's value exactly;
    a window at least the length changes nothing; otherwise the attention of
    the last W rows (scipy softmax)."""
    import scipy.special

    lay, s, c32, table, lens, cache, q, K, V = _tiny_cache("turboquant_k3v4_nc", lens=(37, 5))
    qd = q
    full = O.decode(lay, qd, cache, table, lens, s, c32, 0.25)
    np.testing.assert_array_equal(O.decode(lay, qd, cache, table, lens, s, c32, 0.25, sliding_window=37)[0], full[0])
    np.testing.assert_array_equal(O.decode(lay, qd, cache, table, lens, s, c32, 0.25, sliding_window=1000)[0], full[0])
    one, lse1 = O.decode(lay, qd, cache, table, lens, s, c32, 0.25, sliding_window=1)
    R = O.rotation(np.asarray(s, np.float64))
    g = qd.shape[1] // cache.shape[2]
    for b, L in enumerate(lens):
        for hq in range(qd.shape[1]):
            Kd, Vd = O.gather_sequence(lay, cache, table[b], int(L), hq // g, c32)
            np.testing.assert_array_equal(one[b, hq], Vd[L - 1])
            np.testing.assert_allclose(lse1[b, hq], 0.25 * Kd[L - 1] @ (R @ qd[b, hq]), rtol=1e-12)
            for W in (3, 16, 17):
                o, l = O.decode(lay, qd, cache, table, lens, s, c32, 0.25, rows=[(b, hq)], sliding_window=W)
                sc = 0.25 * (Kd[max(0, L - W):] @ (R @ qd[b, hq]))
                np.testing.assert_allclose(o[b, hq], scipy.special.softmax(sc) @ Vd[max(0, L - W):], rtol=1e-11)
                np.testing.assert_allclose(l[b, hq], scipy.special.logsumexp(sc), rtol=1e-12)


# ---------------------------------------------------------------- sparse-V gate


def test_sparse_v_gate_closed_form():
    """Two tokens with scores 8 and 0 (factor e^-8 = 3.4e-4 < 1e-3): the gate
    drops token 2's value but keeps its weight in the denominator, so
    o = v1 / (1 + e^-8) while exact attention is (v1 + e^-8 v2) / (1 + e^-8);
    the lse is exact; the bound is e^-8 |v2| / (1 + e^-8).  A gate below
    every factor is exact attention with a zero bound."""
    q = np.array([1.0, 0.0])
    K = np.array([[8.0, 0.0], [0.0, 0.0]])
    V = np.array([[1.0, 2.0], [-3.0, 5.0]])
    e = math.exp(-8.0)
    o, lse, b = O.attend_sparse_v(q, K, V, 1.0, 1e-3)
    np.testing.assert_allclose(o, V[0] / (1 + e), rtol=1e-15)
    assert lse == pytest.approx(8 + math.log1p(e), abs=1e-14)
    np.testing.assert_allclose(b, e * np.abs(V[1]) / (1 + e), rtol=1e-14)
    ox, lx = O.attend(q, K, V, 1.0)
    np.testing.assert_allclose(np.abs(o - ox), b, rtol=1e-12)  # the bound is tight here
    o0, lse0, b0 = O.attend_sparse_v(q, K, V, 1.0, e / 2)
    np.testing.assert_allclose(o0, ox, rtol=1e-15)
    assert lse0 == lx and np.all(b0 == 0)
    # a sink joins the denominator only: o = v1 / (1 + e^-8 + e^{sink - 8})
    o, lse, b = O.attend_sparse_v(q, K, V, 1.0, 1e-3, sink=7.0)
    np.testing.assert_allclose(o, V[0] / (1 + e + math.exp(-1.0)), rtol=1e-15)


def test_sparse_v_bound_covers_every_subset_of_gated_tokens():
    """A kernel gates against a running maximum, which never exceeds the
    final one, so it drops some subset of the tokens gated here: every such
    result stays within the bound of exact attention."""
    rng = np.random.default_rng(4)
    for trial in range(20):
        n, d = 200, 16
        q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d))
        scale, gate = 1.0, 10.0 ** rng.uniform(-4, -1)
        ox, _ = O.attend(q, K, V, scale)
        _, _, b = O.attend_sparse_v(q, K, V, scale, gate)
        s = scale * (K @ q)
        f = np.exp(s - s.max())
        gated = np.flatnonzero(f < gate)
        assert len(gated) > 0
        for _ in range(5):
            sub = gated[rng.random(len(gated)) < 0.5]
            keep = np.ones(n, bool)
            keep[sub] = False
            o_sub = (f[keep] @ V[keep]) / f.sum()
            assert np.all(np.abs(o_sub - ox) <= b * (1 + 1e-12) + 1e-15)
