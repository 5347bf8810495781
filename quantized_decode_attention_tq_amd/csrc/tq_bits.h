// Bit-level helpers of the kernels: FP8 E4M3 encoding, byte permutes and the
// unpacking of packed key/value codes into MFMA operand registers.
//
// Everything here is plain integer/float code that also compiles for the
// host, where the two AMDGPU byte-permute instructions are emulated, so the
// unpacking logic is unit-tested on the CPU against the oracle's packing
// (through the host build of the probe library, csrc/tests/tq_probe.hip).
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

#if defined(__HIPCC__)
#define TQ_HD __host__ __device__ __forceinline__
#else
#define TQ_HD inline
#endif

namespace tq {

TQ_HD uint32_t f32_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return u;
}

// v_perm_b32: byte k of the result is byte sel[k] of the 8-byte value
// {s0 (bytes 4..7), s1 (bytes 0..3)}; selector 12 gives 0x00, >= 13 gives 0xFF.
TQ_HD uint32_t perm32(uint32_t s0, uint32_t s1, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(s0, s1, sel);
#else
  uint64_t v = (static_cast<uint64_t>(s0) << 32) | s1;
  uint32_t r = 0;
  for (int k = 0; k < 4; ++k) {
    uint32_t b = (sel >> (8 * k)) & 0xFF, byte;
    if (b < 8)
      byte = static_cast<uint32_t>(v >> (8 * b)) & 0xFF;
    else if (b == 12)
      byte = 0;
    else if (b >= 13)
      byte = 0xFF;
    else
      byte = ((v >> (16 * (b - 8) + 15)) & 1) ? 0xFF : 0;
    r |= byte << (8 * k);
  }
  return r;
#endif
}

// v_alignbyte_b32: low dword of {hi, lo} >> (8 * (shift & 3)).
TQ_HD uint32_t alignbyte(uint32_t hi, uint32_t lo, uint32_t shift) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_alignbyte(hi, lo, shift);
#else
  return static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> (8 * (shift & 3)));
#endif
}

// ---------------------------------------------------------------------------
// FP8 E4M3 (OCP "fn": bias 7, no infinities, S.1111.111 = NaN) from fp32,
// round to nearest even, saturating at +-448; NaN -> 0x7F.
// ---------------------------------------------------------------------------
TQ_HD uint32_t f32_to_e4m3(float x) {
  const uint32_t u = f32_bits(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;           // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;   // |x| >= 448 (and inf): saturate
  if (a >= 0x3C800000u) {                      // |x| >= 2^-6: normal E4M3
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
    return sign | (r - (120u << 3));           // rebias exponent 127 -> 7
  }
  // subnormal range: value = m * 2^-9, m = rne(|x| * 512) in 0..8 (8 = 2^-6)
  float ax = std::fabs(x) * 512.0f;
  return sign | static_cast<uint32_t>(rintf(ax));
}

// ---------------------------------------------------------------------------
// Key codebook lookup: codes -> fp16 centroids, two per dword, via v_perm.
// The fp16 centroid table is split into its low and high bytes; an 8-entry
// byte table fits the two source dwords of one permute.
// ---------------------------------------------------------------------------
struct Lut8 {
  uint32_t lo0, lo1, hi0, hi1;  // low/high bytes of fp16 centroid 0..3 / 4..7
};

// S: four 3-bit codes, one per byte (values 0..7).  out0 = fp16 pair
// (c[S.b0], c[S.b1]), out1 = (c[S.b2], c[S.b3]).
TQ_HD void lut8(uint32_t S, const Lut8& t, uint32_t& out0, uint32_t& out1) {
  uint32_t lo = perm32(t.lo1, t.lo0, S);
  uint32_t hi = perm32(t.hi1, t.hi0, S);
  out0 = perm32(hi, lo, 0x05010400u);
  out1 = perm32(hi, lo, 0x07030602u);
}

// 16 entries: two 8-entry tables, picked per byte by bit 3 of the code.
TQ_HD void lut16(uint32_t S, const Lut8& a, const Lut8& b, uint32_t& out0, uint32_t& out1) {
  uint32_t s7 = S & 0x07070707u;
  uint32_t m = ((S >> 3) & 0x01010101u) * 0xFFu;
  uint32_t lo = (m & perm32(b.lo1, b.lo0, s7)) | (~m & perm32(a.lo1, a.lo0, s7));
  uint32_t hi = (m & perm32(b.hi1, b.hi0, s7)) | (~m & perm32(a.hi1, a.hi0, s7));
  out0 = perm32(hi, lo, 0x05010400u);
  out1 = perm32(hi, lo, 0x07030602u);
}

// 32 packed 3-bit key codes (12 bytes, LSB-first bit stream: code j at bits
// 3j..3j+2; bytes 3g..3g+2 hold codes 8g..8g+7) -> eight selector dwords.
// sel[m] holds, in byte g, code 8g + m.  The codes of one byte column are
// gathered first (X = byte 0 of every 3-byte group, Y = byte 1, Z = byte 2),
// then each code is one shift and mask (two for the codes that straddle).
TQ_HD void key3_selectors(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t sel[8]) {
  uint32_t X = perm32(w2, perm32(w1, w0, 0x00060300u), 0x05020100u);
  uint32_t Y = perm32(w2, perm32(w1, w0, 0x00070401u), 0x06020100u);
  uint32_t Z = perm32(w2, perm32(w1, w0, 0x00000502u), 0x07040100u);
  sel[0] = X & 0x07070707u;
  sel[1] = (X >> 3) & 0x07070707u;
  sel[2] = ((X >> 6) & 0x03030303u) | ((Y << 2) & 0x04040404u);
  sel[3] = (Y >> 1) & 0x07070707u;
  sel[4] = (Y >> 4) & 0x07070707u;
  sel[5] = ((Y >> 7) & 0x01010101u) | ((Z << 1) & 0x06060606u);
  sel[6] = (Z >> 2) & 0x07070707u;
  sel[7] = (Z >> 5) & 0x07070707u;
}

// 3-bit Lloyd-Max value codes of 4 tokens -> eight selector dwords for the
// codebook lookup: w[g] holds token g's 8 codes in bits 0..23 (its lane
// column of dims); sel[m] holds, in byte g, token g's code m.  The four
// 24-bit words joined end to end are a 32-code stream whose code 8g + m is
// token g's code m, which key3_selectors lays out exactly so.
TQ_HD void lm_value_selectors(const uint32_t w[4], uint32_t sel[8]) {
  const uint32_t s0 = perm32(w[1], w[0], 0x04020100u);  // t0 bytes 0..2, t1 byte 0
  const uint32_t s1 = perm32(w[2], w[1], 0x05040201u);  // t1 bytes 1..2, t2 bytes 0..1
  const uint32_t s2 = perm32(w[3], w[2], 0x06050402u);  // t2 byte 2, t3 bytes 0..2
  key3_selectors(s0, s1, s2, sel);
}

// 3-bit keys, two dims per lookup: the lane's 32 codes are a 96-bit
// LSB-first stream {w2:w1:w0}; the 6-bit field at bit 6j holds the codes of
// dims 2j (bits 0..2) and 2j + 1 (bits 3..5), and indexes a 64-entry table
// whose entry f is the fp16 pair (c[f & 7], c[f >> 3]).  Fields 5 and 10
// straddle a dword boundary.
TQ_HD uint32_t key3_pair_field(uint32_t w0, uint32_t w1, uint32_t w2, int j) {
  const int b = 6 * j;
  if (b + 6 <= 32) return (w0 >> b) & 63u;
  if (b < 32) return ((w0 >> b) | (w1 << (32 - b))) & 63u;
  if (b + 6 <= 64) return (w1 >> (b - 32)) & 63u;
  if (b < 64) return ((w1 >> (b - 32)) | (w2 << (64 - b))) & 63u;
  return (w2 >> (b - 64)) & 63u;
}
// The same field at bits 8..13 of a 32-bit window of the stream (other bits
// hold neighbouring codes): one shift or funnel shift, so that (window &
// 0x3F00) is the field times a 256-byte table stride.
TQ_HD uint32_t key3_pair_window(uint32_t w0, uint32_t w1, uint32_t w2, int j) {
  const int s = 6 * j - 8;  // stream bit at window bit 0
  if (s < 0) return w0 << (-s);
  if (s >= 64) return w2 >> (s - 64);
  const uint32_t lo = s < 32 ? w0 : w1, hi = s < 32 ? w1 : w2;
  const int r = s & 31;
  return r == 0 ? lo : ((lo >> r) | (hi << (32 - r)));
}
// Table entry f of the pair lookup: fp16 bits of c[f & 7] (low half) and
// c[f >> 3] (high half), from the 8-entry fp16 codebook h.
TQ_HD uint32_t key3_pair_entry(const uint16_t h[8], int f) {
  return static_cast<uint32_t>(h[f & 7]) | (static_cast<uint32_t>(h[f >> 3]) << 16);
}
// The pair lookup's MFMA operand order: dword j of the lane's 16 holds dims
// 2j, 2j + 1, so chunk c element e holds dim 8c + e.
TQ_HD int key3_pair_dim(int c, int e) { return 8 * c + e; }

// The same for 4-bit Lloyd-Max value codes: w[g] holds token g's 8 codes
// (dim 8r + m at bits 4m); sel[m] holds, in byte g, token g's code m (0..15).
// Bytes k of the four words are gathered into one dword (two permutes per
// pair of words, then one across the pairs), then split into nibbles.
TQ_HD void lm4_value_selectors(const uint32_t w[4], uint32_t sel[8]) {
  const uint32_t a = perm32(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t b = perm32(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t c = perm32(w[3], w[2], 0x05010400u);
  const uint32_t d = perm32(w[3], w[2], 0x07030602u);
  const uint32_t x[4] = {perm32(c, a, 0x05040100u), perm32(c, a, 0x07060302u), perm32(d, b, 0x05040100u),
                         perm32(d, b, 0x07060302u)};  // x[k] byte g = byte k of w[g]
  for (int k = 0; k < 4; ++k) {
    sel[2 * k] = x[k] & 0x0F0F0F0Fu;
    sel[2 * k + 1] = (x[k] >> 4) & 0x0F0F0F0Fu;
  }
}

// 2-bit Lloyd-Max value codes: w[g] holds token g's 8 codes in bits 0..15
// (dim 8r + m at bits 2m; bits 16..31 are not codes); sel[m] holds, in byte
// g, token g's code m (0..3).
TQ_HD void lm2_value_selectors(const uint32_t w[4], uint32_t sel[8]) {
  const uint32_t a = perm32(w[1], w[0], 0x05010400u);
  const uint32_t c = perm32(w[3], w[2], 0x05010400u);
  const uint32_t x0 = perm32(c, a, 0x05040100u), x1 = perm32(c, a, 0x07060302u);
  for (int m = 0; m < 8; ++m) sel[m] = ((m < 4 ? x0 : x1) >> (2 * (m & 3))) & 0x03030303u;
}

// Order of the 32 key dims of a 3-bit lane chunk in the MFMA operand: chunk c
// (0..3) element e (0..7) holds dim 8*(e & 3) + 2c + (e >> 2).
TQ_HD int key3_dim(int c, int e) { return 8 * (e & 3) + 2 * c + (e >> 2); }

// 4-bit keys: dword k of a lane chunk holds dims 8k..8k+7 (low nibble =
// even dim).  lo = w & 0x0F0F0F0F selects the even dims, hi the odd ones.
// Chunk c element e holds dim 8c + (e < 4 ? 2e : 2(e - 4) + 1).
TQ_HD int key4_dim(int c, int e) { return 8 * c + (e < 4 ? 2 * e : 2 * (e - 4) + 1); }

// 2-bit keys: a lane chunk is 2 dwords, byte b of dword w holding dims
// 16w + 4b .. 16w + 4b + 3 (code k of the byte at bits 2k).  Selector
// (w >> 2k) & 0x03030303 holds dim 16w + 4b + k in byte b; chunk c takes
// selectors k = 2(c & 1) and k + 1 of dword c >> 1, so element e holds dim
// 16(c >> 1) + 4(e & 3) + 2(c & 1) + (e >> 2).
TQ_HD uint32_t key2_selector(uint32_t w, int k) { return (w >> (2 * k)) & 0x03030303u; }
TQ_HD int key2_dim(int c, int e) { return 16 * (c >> 1) + 4 * (e & 3) + 2 * (c & 1) + (e >> 2); }

// ---------------------------------------------------------------------------
// Value codes -> fp16 MFMA operand pairs, as fp16 subnormals.
//
// A 16-bit half whose exponent field is zero is the subnormal mantissa *
// 2^-24, i.e. linear in its bits: a code sitting at bit position p (p + width
// <= 10) of an otherwise zero half is exactly code * 2^(p-24).  Masking the
// code in place therefore yields an MFMA operand with no conversion; the
// power-of-two factor is undone after the accumulation.  Each output dword
// holds the same dim of two tokens (token a in the low half).
// ---------------------------------------------------------------------------

// 4-bit: wa, wb = the dword of dims 8r..8r+7 of tokens a and b.  out[n]
// (n = 0..7) = dim 8r+n of (a, b); code at bit position (n & 1) * 4.
// The unpack is split into a per-pair step (interleave the two tokens'
// bytes: val4_pre / val3_pre) and a one-mask step per output
// (val4_get / val3_get), so a caller can keep only the interleaved words
// and produce each output when it is consumed.
struct Val4Pre {
  uint32_t w[4];  // p0, q0 = p0 >> 8, p1, q1 = p1 >> 8
};
TQ_HD Val4Pre val4_pre(uint32_t wa, uint32_t wb) {
  Val4Pre r;
  r.w[0] = perm32(wb, wa, 0x05040100u);  // bits 0..15 of a | bits 0..15 of b
  r.w[2] = perm32(wb, wa, 0x07060302u);  // bits 16..31
  r.w[1] = r.w[0] >> 8;
  r.w[3] = r.w[2] >> 8;
  return r;
}
TQ_HD uint32_t val4_get(const Val4Pre& r, int n) { return r.w[n >> 1] & ((n & 1) ? 0x00F000F0u : 0x000F000Fu); }

TQ_HD void val4_pairs(uint32_t wa, uint32_t wb, uint32_t out[8]) {
  const Val4Pre r = val4_pre(wa, wb);
  for (int n = 0; n < 8; ++n) out[n] = val4_get(r, n);
}
TQ_HD int val4_pos(int n) { return (n & 1) * 4; }

// 3-bit: wa, wb = 24 bits (bytes 0..2) = dims 8r..8r+7, code m at bits 3m.
// out[m] = dim 8r+m of (a, b); code at bit position val3_pos(m).
struct Val3Pre {
  uint32_t w[3];  // word bits 0..15, 8..23, 16..23 of a | the same of b
};
TQ_HD Val3Pre val3_pre(uint32_t wa, uint32_t wb) {
  Val3Pre r;
  r.w[0] = perm32(wb, wa, 0x05040100u);
  r.w[1] = perm32(wb, wa, 0x06050201u);
  r.w[2] = perm32(wb, wa, 0x0C060C02u);
  return r;
}
TQ_HD uint32_t val3_get(const Val3Pre& r, int m) {
  constexpr uint32_t kMask[8] = {0x00070007u, 0x00380038u, 0x01C001C0u, 0x000E000Eu,
                                 0x00700070u, 0x03800380u, 0x001C001Cu, 0x00E000E0u};
  return r.w[m < 3 ? 0 : (m < 6 ? 1 : 2)] & kMask[m];
}

TQ_HD void val3_pairs(uint32_t wa, uint32_t wb, uint32_t out[8]) {
  const Val3Pre r = val3_pre(wa, wb);
  for (int m = 0; m < 8; ++m) out[m] = val3_get(r, m);
}
// code m starts at bit 3m of the word and its window starts at bit 8*floor(3m/8)
TQ_HD int val3_pos(int m) { return (3 * m) & 7; }

// 2-bit: wa, wb = 16 bits (bytes 0..1) = dims 8r..8r+7, code m at bits 2m.
// out[m] = dim 8r+m of (a, b); code at bit position val2_pos(m) (codes 4..7
// come from the word shifted down a byte, so no code reaches the exponent).
struct Val2Pre {
  uint32_t w[2];  // word bits 0..15 of a | of b; the same shifted right by 8
};
TQ_HD Val2Pre val2_pre(uint32_t wa, uint32_t wb) {
  Val2Pre r;
  r.w[0] = perm32(wb, wa, 0x05040100u);
  r.w[1] = r.w[0] >> 8;
  return r;
}
TQ_HD uint32_t val2_get(const Val2Pre& r, int m) { return r.w[m >> 2] & (0x00030003u << (2 * (m & 3))); }

TQ_HD void val2_pairs(uint32_t wa, uint32_t wb, uint32_t out[8]) {
  const Val2Pre r = val2_pre(wa, wb);
  for (int m = 0; m < 8; ++m) out[m] = val2_get(r, m);
}
TQ_HD int val2_pos(int m) { return 2 * (m & 3); }

}  // namespace tq
