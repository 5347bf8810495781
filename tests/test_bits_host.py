"""The kernels' bit helpers (FP8 encode, codebook lookup by byte permute,
3-bit selector extraction, value-code operand packing), run through their
host build, against the oracle's packing and number formats.  CPU only."""

import numpy as np
import pytest

import oracle as O
import probe

RNG = np.random.default_rng(2024)


def _bytes_to_words(b):
    b = np.asarray(b, np.uint8)
    pad = (-b.shape[-1]) % 4
    b = np.concatenate([b, np.zeros(b.shape[:-1] + (pad,), np.uint8)], axis=-1)
    return b.view(np.uint32)


def test_perm_semantics_hand_cases():
    s0, s1 = 0x44332211, 0x88776655
    cases = [(0x03020100, 0x88776655), (0x07060504, 0x44332211), (0x0C0D0C0D, 0x00FF00FF), (0x04000400, 0x11551155)]
    got = probe.bits_host("perm", np.array([[s0, s1, sel] for sel, _ in cases], np.uint32))[:, 0]
    np.testing.assert_array_equal(got, [w for _, w in cases])


def test_alignbyte_hand_cases():
    got = probe.bits_host("alignbyte", np.array([[0xDDCCBBAA, 0x44332211, s] for s in range(4)], np.uint32))[:, 0]
    np.testing.assert_array_equal(got, [0x44332211, 0xAA443322, 0xBBAA4433, 0xCCBBAA44])


def test_f32_to_e4m3_all_16bit_inputs():
    for dtype in ("bf16", "f16"):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        x = O.widen(bits, dtype)
        f32 = x.astype(np.float32).view(np.uint32)
        got = probe.bits_host("f32_to_e4m3", f32[:, None])[:, 0]
        want = O.fp8_e4m3fn_encode(x).astype(np.uint32)
        np.testing.assert_array_equal(got, want)


def test_key3_selectors_match_oracle_packing():
    codes = RNG.integers(0, 8, (4000, 32))
    packed = O.pack_lsb(codes, 3)  # (n, 12) bytes
    w = _bytes_to_words(packed)
    sel = probe.bits_host("key3_selectors", w)
    sb = sel.view(np.uint8).reshape(-1, 8, 4)  # [item][m][g] = code 8g + m
    for m in range(8):
        for g in range(4):
            np.testing.assert_array_equal(sb[:, m, g], codes[:, 8 * g + m])


def test_key3_pair_fields_match_oracle_packing():
    """Field j of a lane's 96-bit stream = code of dim 2j | code of dim 2j+1 << 3
    (fields 5 and 10 straddle a dword)."""
    codes = RNG.integers(0, 8, (4000, 32))
    w = _bytes_to_words(O.pack_lsb(codes, 3))  # (n, 3)
    for half in (0, 1):
        inp = np.column_stack([w, np.full(len(w), half, np.uint32)])
        got = probe.bits_host("key3_pair_fields", inp)
        for k in range(8):
            j = 8 * half + k
            np.testing.assert_array_equal(got[:, k], codes[:, 2 * j] | (codes[:, 2 * j + 1] << 3))
        win = probe.bits_host("key3_pair_windows", inp)
        np.testing.assert_array_equal((win >> 8) & 63, got)


def test_key3_pair_entries_hold_both_centroids():
    c3, _ = O.codebook_tables(128, 3)
    h = np.asarray(c3, np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    for f0 in range(0, 64, 8):
        got = probe.bits_host("key3_pair_entries", np.concatenate([h, [f0]]).astype(np.uint32)[None, :])[0]
        for k in range(8):
            f = f0 + k
            assert got[k] & 0xFFFF == h[f & 7] and got[k] >> 16 == h[f >> 3]


def _f16_table(vals):
    h = np.asarray(vals, np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    lo = h & 0xFF
    hi = h >> 8
    def pack(v, base):
        return v[base] | (v[base + 1] << 8) | (v[base + 2] << 16) | (v[base + 3] << 24)
    return h, [pack(lo, 0), pack(lo, 4), pack(hi, 0), pack(hi, 4)]


def test_lut8_and_lut16():
    c3, _ = O.codebook_tables(128, 3)
    h3, t3 = _f16_table(c3)
    codes = RNG.integers(0, 8, (3000, 4))
    S = (codes[:, 0] | (codes[:, 1] << 8) | (codes[:, 2] << 16) | (codes[:, 3] << 24)).astype(np.uint32)
    out = probe.bits_host("lut8", np.column_stack([S] + [np.full(len(S), t, np.uint32) for t in t3]))
    halves = out[:, :2].view(np.uint16).reshape(-1, 4)
    np.testing.assert_array_equal(halves, h3[codes])

    c4, _ = O.codebook_tables(128, 4)
    h4a, ta = _f16_table(c4[:8])
    h4b, tb = _f16_table(c4[8:])
    h4 = np.concatenate([h4a, h4b])
    codes = RNG.integers(0, 16, (3000, 4))
    S = (codes[:, 0] | (codes[:, 1] << 8) | (codes[:, 2] << 16) | (codes[:, 3] << 24)).astype(np.uint32)
    out = probe.bits_host("lut16", np.column_stack([S] + [np.full(len(S), t, np.uint32) for t in ta + tb]))
    halves = out[:, :2].view(np.uint16).reshape(-1, 4)
    np.testing.assert_array_equal(halves, h4[codes])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_pairs_are_subnormal_codes(bits):
    """Each output half is code << pos, i.e. the fp16 subnormal code * 2^(pos-24)."""
    n = 3000
    ca = RNG.integers(0, 1 << bits, (n, 8))
    cb = RNG.integers(0, 1 << bits, (n, 8))
    wa = _bytes_to_words(O.pack_lsb(ca, bits))[:, 0]
    wb = _bytes_to_words(O.pack_lsb(cb, bits))[:, 0]
    out = probe.bits_host({2: "val2_pairs", 3: "val3_pairs", 4: "val4_pairs"}[bits], np.column_stack([wa, wb]))
    pos = {2: [2 * (m & 3) for m in range(8)], 3: [(3 * m) & 7 for m in range(8)],
           4: [(m & 1) * 4 for m in range(8)]}[bits]
    for m in range(8):
        lo = out[:, m] & 0xFFFF
        hi = out[:, m] >> 16
        np.testing.assert_array_equal(lo, ca[:, m] << pos[m])
        np.testing.assert_array_equal(hi, cb[:, m] << pos[m])
        assert np.all(lo < 0x400) and np.all(hi < 0x400)  # exponent field zero: subnormal or zero
        vals = lo.astype(np.uint16).view(np.float16).astype(np.float64)
        np.testing.assert_array_equal(vals, ca[:, m] * 2.0 ** (pos[m] - 24))


def test_key2_selectors_put_one_code_per_byte():
    """Selector k of a dword of 16 packed 2-bit codes holds, in byte b, the
    code of dim 4b + k (the order the decode's 2-bit key operand takes)."""
    codes = RNG.integers(0, 4, (3000, 16))
    w = _bytes_to_words(O.pack_lsb(codes, 2))[:, 0]
    out = probe.bits_host("key2_selectors", w[:, None])
    for k in range(4):
        for b in range(4):
            np.testing.assert_array_equal((out[:, k] >> (8 * b)) & 0xFF, codes[:, 4 * b + k])


def test_lm_value_selectors_transpose_four_tokens():
    """Four tokens' 3-bit code words (8 codes each, bits 0..23, garbage in
    bits 24..31) -> selector m holds token g's code m in byte g."""
    codes = RNG.integers(0, 8, (3000, 4, 8))
    w = np.stack([_bytes_to_words(np.concatenate([O.pack_lsb(codes[:, g], 3),
                                                  RNG.integers(0, 256, (3000, 1)).astype(np.uint8)], axis=1))[:, 0]
                  for g in range(4)], axis=1)
    out = probe.bits_host("lm_value_selectors", w)
    for m in range(8):
        for g in range(4):
            np.testing.assert_array_equal((out[:, m] >> (8 * g)) & 0xFF, codes[:, g, m])


@pytest.mark.parametrize("bits", [4, 2])
def test_lm_value_selectors_at_4_and_2_bits(bits):
    """Four tokens' 4-bit (32-bit words) or 2-bit (bits 0..15, garbage above)
    Lloyd-Max code words -> selector m holds token g's code m in byte g."""
    codes = RNG.integers(0, 1 << bits, (3000, 4, 8))
    nbytes = 8 * bits // 8
    w = np.stack([_bytes_to_words(np.concatenate([O.pack_lsb(codes[:, g], bits),
                                                  RNG.integers(0, 256, (3000, 4 - nbytes)).astype(np.uint8)],
                                                 axis=1))[:, 0]
                  for g in range(4)], axis=1)
    out = probe.bits_host(f"lm{bits}_value_selectors", w)
    for m in range(8):
        for g in range(4):
            np.testing.assert_array_equal((out[:, m] >> (8 * g)) & 0xFF, codes[:, g, m])
