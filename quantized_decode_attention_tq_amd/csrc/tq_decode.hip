// tq_decode_attention: split-KV decode attention over the compressed paged
// cache ([PR] "实现拆解" item 4: stage 1 scores and accumulates values per
// split, stage 2 merges the splits with a log-sum-exp reduction; [API]
// _decode_attention).
//
// Stage 1 work unit: one workgroup per (sequence b, KV head hk, group of up
// to 16 query heads, split s); its 4 wave64s take the split's 16-token tiles
// round-robin and merge in LDS at the end.  Per tile a wave:
//   - builds the key tile (16 tokens x 128 dims) as fp16 MFMA operands: FP8
//     keys by the hardware FP8->fp16 convert, Lloyd-Max codes through a
//     v_perm byte lookup of the fp16 codebook;
//   - scores S^T = K . Q^T with 4 MFMA 16x16x32 f16 (tokens on rows, query
//     heads on columns), the query rotated by the same transform and
//     pre-scaled by scale*log2(e) (MSE presets, [API] _decode_attention);
//   - applies the per-token key norm, an online softmax in base 2, and
//   - accumulates O^T = V^T . P^T with 8 MFMA 16x16x16 f16, the value codes
//     entering as fp16 subnormals (no conversion) and the per-token value
//     scale folded into P; the per-token zero point is accumulated on the
//     VALU as sum(p * zero).
// The GQA group rides on the MFMA's 16 columns, so the key/value bytes of a
// (token, KV head) are read and decoded once for all its query heads.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>

#include "tq.h"
#include "tq_bits.h"
#include "tq_internal.h"

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));

// Slot geometry per preset at head_dim 128 (see tq_layout_init).
template <int P>
struct Preset;
template <>
struct Preset<TQ_K8V4> {
  static constexpr int kFp8 = 1, kKb = 8, kVb = 4, kKdata = 128, kKps = 128, kVdata = 64, kSlot = 196;
};
template <>
struct Preset<TQ_4BIT_NC> {
  static constexpr int kFp8 = 0, kKb = 4, kVb = 4, kKdata = 64, kKps = 66, kVdata = 64, kSlot = 134;
};
template <>
struct Preset<TQ_K3V4_NC> {
  static constexpr int kFp8 = 0, kKb = 3, kVb = 4, kKdata = 48, kKps = 50, kVdata = 64, kSlot = 118;
};
template <>
struct Preset<TQ_3BIT_NC> {
  static constexpr int kFp8 = 0, kKb = 3, kVb = 3, kKdata = 48, kKps = 50, kVdata = 48, kSlot = 102;
};

// The constants above follow the slot layout of tq_layout_init at head_dim 128.
template <int P>
constexpr bool preset_geometry_ok() {
  using T = Preset<P>;
  return T::kKdata == (T::kFp8 ? kD : kD * T::kKb / 8) && T::kKps == (T::kFp8 ? kD : T::kKdata + 2) &&
         T::kVdata == kD * T::kVb / 8 && T::kSlot == ((T::kKps + T::kVdata + 4 + 1) / 2) * 2;
}
static_assert(preset_geometry_ok<TQ_K8V4>() && preset_geometry_ok<TQ_4BIT_NC>() &&
                  preset_geometry_ok<TQ_K3V4_NC>() && preset_geometry_ok<TQ_3BIT_NC>(),
              "slot geometry");

struct DecodeArgs {
  const uint16_t* query;
  const uint8_t* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* signs;
  const float* centroids;
  float* partials;  // [B][Hq][S][D+1]
  float qscale;     // softmax scale * log2(e)
  int32_t q_bf16;
  int32_t num_q_heads, num_kv_heads, group, head_groups, heads_per_wg;
  int32_t block_size, bt_stride, num_splits;
};

__device__ __forceinline__ float widen16(uint32_t bits, bool bf16) {
  if (bf16) return __uint_as_float(bits << 16);
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs; remap
// so that consecutive *logical* ids (the KV heads of one sequence/split,
// which share cache lines) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, loc = bid / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + loc;
}

// dword from a 2-byte aligned address: two aligned dwords, realigned.
__device__ __forceinline__ uint32_t ld32_u(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const u32x2a4 w = *reinterpret_cast<const u32x2a4*>(a & ~static_cast<uintptr_t>(3));
  return tq::alignbyte(w.y, w.x, static_cast<uint32_t>(a & 3));
}

__device__ __forceinline__ uint32_t ld16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// Position of query dim d in the fp16 query operand image: lane quarter q,
// MFMA chunk c, element e -> q*32 + c*8 + e, matching the order in which the
// key operand holds dims (FP8 keys: quarter q loads dims 16q..16q+15 and
// 64+16q..64+16q+15; 4-bit keys: even dims then odd dims of each byte group;
// 3-bit keys: the selector order of tq::key3_selectors).
template <int P>
__device__ __forceinline__ int qh_pos(int d) {
  using T = Preset<P>;
  if (T::kFp8) {
    const int r = d & 63;
    return (r >> 4) * 32 + ((d >> 6) * 2 + ((r & 15) >> 3)) * 8 + (d & 7);
  }
  const int q = d >> 5, dd = d & 31;
  if (T::kKb == 4) {
    const int r = dd & 7;
    return q * 32 + (dd >> 3) * 8 + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
  }
  return q * 32 + ((dd & 7) >> 1) * 8 + (dd & 1) * 4 + (dd >> 3);
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4a4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half4 as_half4(uint32_t a, uint32_t b) {
  u32x2a4 v = {a, b};
  return __builtin_bit_cast(half4, v);
}
__device__ __forceinline__ uint32_t h2_bits(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Byte offsets (lane constants) of what one lane loads for a 16-token tile,
// relative to the tile's first slot row.  Block bases and the tile's first
// row are multiples of 32 bytes, so the alignment of every address is a lane
// constant too: unaligned fields are read as aligned dwords and realigned.
template <int P>
struct LaneOff {
  uint32_t k, ksh;  // aligned-down key chunk start, its misalignment
  uint32_t meta0;   // slot start of token 4q (token 4q+i is i rows further)
  uint32_t vcol;    // byte offset of the lane's value-code column inside a slot
};

// Registers one tile's loads land in.
template <int P>
struct TileRegs {
  uint32_t k[8];
  uint32_t v[4][2];
  uint32_t sz[4];  // fp16 scale | fp16 zero << 16
  uint32_t gm[4];  // fp16 key norm (MSE keys)
};

template <int P>
__device__ __forceinline__ LaneOff<P> lane_offsets(int hl, int q4, int hk, int Hk) {
  using T = Preset<P>;
  LaneOff<P> o;
  const uint32_t kraw = static_cast<uint32_t>((hl * Hk + hk) * T::kSlot) +
                        static_cast<uint32_t>(T::kFp8 ? 16 * q4 : (T::kKb == 4 ? 16 * q4 : 12 * q4));
  o.k = kraw & ~3u;
  o.ksh = kraw & 3u;
  o.meta0 = static_cast<uint32_t>((4 * q4 * Hk + hk) * T::kSlot);
  o.vcol = static_cast<uint32_t>(T::kKps + (T::kVb == 4 ? 4 * hl : 3 * hl));
  return o;
}

// Issue every load of one tile.  tb: the tile's first slot row (uniform);
// row: bytes per token row (Hk * slot, uniform).
template <int P>
__device__ __forceinline__ void load_tile(const uint8_t* tb, uint32_t row, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
  if constexpr (T::kFp8 != 0) {
    const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(tb + o.k);
    const u32x4a4 k1 = *reinterpret_cast<const u32x4a4*>(tb + o.k + 64);
    r.k[0] = k0.x; r.k[1] = k0.y; r.k[2] = k0.z; r.k[3] = k0.w;
    r.k[4] = k1.x; r.k[5] = k1.y; r.k[6] = k1.z; r.k[7] = k1.w;
  } else {
    const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(tb + o.k);
    r.k[0] = k0.x; r.k[1] = k0.y; r.k[2] = k0.z; r.k[3] = k0.w;
    if (T::kKb == 4) r.k[4] = *reinterpret_cast<const uint32_t*>(tb + o.k + 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // value codes of token 4q+i; the row stride may be 2 mod 4, so the
    // whole in-tile offset is aligned down (tile bases are 32-byte aligned)
    const uint32_t vo = i * row + o.meta0 + o.vcol;
    if constexpr (T::kSlot % 4 == 0 && T::kKps % 4 == 0 && T::kVb == 4) {
      r.v[i][0] = *reinterpret_cast<const uint32_t*>(tb + vo);
    } else {
      const u32x2a4 w = *reinterpret_cast<const u32x2a4*>(tb + (vo & ~3u));
      r.v[i][0] = w.x;
      r.v[i][1] = w.y;
    }
    const uint8_t* m = tb + i * row + o.meta0;
    if constexpr (T::kSlot % 4 == 0 && (T::kKps + T::kVdata) % 4 == 0) {
      r.sz[i] = *reinterpret_cast<const uint32_t*>(m + T::kKps + T::kVdata);
    } else {
      r.sz[i] = ld16(m + T::kKps + T::kVdata) | (ld16(m + T::kKps + T::kVdata + 2) << 16);
    }
    if constexpr (T::kFp8 == 0) r.gm[i] = ld16(m + T::kKdata);
  }
}

// Key tile operand for one lane (token = lane % 16, its 32 dims of quarter q).
template <int P>
__device__ __forceinline__ void key_operand(const TileRegs<P>& r, uint32_t sh, const tq::Lut8& la,
                                            const tq::Lut8& lb, half8 A[4]) {
  using T = Preset<P>;
  if constexpr (T::kFp8 != 0) {
    uint32_t hv[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hv[2 * i] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.k[i], 1.0f, false));
      hv[2 * i + 1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.k[i], 1.0f, true));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) A[c] = as_half8(hv[4 * c], hv[4 * c + 1], hv[4 * c + 2], hv[4 * c + 3]);
  } else if constexpr (T::kKb == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = tq::alignbyte(r.k[c + 1], r.k[c], sh);
      uint32_t e0, e1, o0, o1;
      tq::lut16(w & 0x0F0F0F0Fu, la, lb, e0, e1);
      tq::lut16((w >> 4) & 0x0F0F0F0Fu, la, lb, o0, o1);
      A[c] = as_half8(e0, e1, o0, o1);
    }
  } else {
    uint32_t sel[8];
    tq::key3_selectors(tq::alignbyte(r.k[1], r.k[0], sh), tq::alignbyte(r.k[2], r.k[1], sh),
                       tq::alignbyte(r.k[3], r.k[2], sh), sel);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t a0, a1, b0, b1;
      tq::lut8(sel[2 * c], la, a0, a1);
      tq::lut8(sel[2 * c + 1], la, b0, b1);
      A[c] = as_half8(a0, a1, b0, b1);
    }
  }
}

// Online-softmax state of one lane: query head lane % 16; the 4 lane quarters
// hold disjoint tokens and share the reference maximum m.
struct Softmax {
  float m, l, z;  // reference max (log2 domain), sum of p, sum of p * zero
};

// Largest growth of p = 2^(s - m) tolerated before the accumulators are
// rescaled; p * value_scale must also stay inside fp16.
constexpr float kLazyRescaleLog2 = 8.0f;

template <int P>
__device__ __forceinline__ void tile_step(const TileRegs<P>& r, const LaneOff<P>& o, uint32_t row,
                                          const tq::Lut8& la, const tq::Lut8& lb, const half8 bq[4], int valid,
                                          Softmax& sm, f32x4 acc[8]) {
  using T = Preset<P>;
  half8 A[4];
  key_operand<P>(r, o.ksh, la, lb, A);
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[c], bq[c], sc, 0, 0, 0);

  float sco[4], sv[4], zv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sco[i] = T::kFp8 ? sc[i] : sc[i] * half_bits_to_f32(r.gm[i]);
    sv[i] = half_bits_to_f32(r.sz[i] & 0xFFFFu);
    zv[i] = half_bits_to_f32(r.sz[i] >> 16);
  }
  const int lane = threadIdx.x & 63;
  if (valid < 16) {  // tail tile: tokens at or past the sequence end drop out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * (lane >> 4) + i >= valid) {
        sco[i] = -INFINITY;
        sv[i] = 0.f;
        zv[i] = 0.f;
      }
    }
  }
  float tmax = fmaxf(fmaxf(sco[0], sco[1]), fmaxf(sco[2], sco[3]));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float m_cand = fmaxf(sm.m, tmax);
  float p[4], ps[4];
  bool redo = __any(tmax > sm.m + kLazyRescaleLog2);
  if (!redo) {
    float pmax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sco[i] - sm.m);
      ps[i] = p[i] * sv[i];
      pmax = fmaxf(pmax, ps[i]);
    }
    redo = __any(pmax > 65504.f);
  }
  if (redo) {  // rescale the accumulators to the new maximum
    const float alpha = __builtin_amdgcn_exp2f(sm.m - m_cand);
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    sm.l *= alpha;
    sm.z *= alpha;
    sm.m = m_cand;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sco[i] - sm.m);
      ps[i] = p[i] * sv[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.l += p[i];
    sm.z = fmaf(p[i], zv[i], sm.z);
  }
  half2v ps01 = {static_cast<_Float16>(ps[0]), static_cast<_Float16>(ps[1])};
  half2v ps23 = {static_cast<_Float16>(ps[2]), static_cast<_Float16>(ps[3])};
  const half4 pv = as_half4(h2_bits(ps01), h2_bits(ps23));

  uint32_t vw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (T::kSlot % 4 == 0 && T::kKps % 4 == 0 && T::kVb == 4)
      vw[i] = r.v[i][0];
    else
      vw[i] = tq::alignbyte(r.v[i][1], r.v[i][0], (i * row + o.meta0 + o.vcol) & 3u);
  }
  uint32_t v01[8], v23[8];
  if (T::kVb == 4) {
    tq::val4_pairs(vw[0], vw[1], v01);
    tq::val4_pairs(vw[2], vw[3], v23);
  } else {
    tq::val3_pairs(vw[0], vw[1], v01);
    tq::val3_pairs(vw[2], vw[3], v23);
  }
#pragma unroll
  for (int n = 0; n < 8; ++n)
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(v01[n], v23[n]), pv, acc[n], 0, 0, 0);
}

// Stage 1.  A workgroup owns (sequence b, group of heads_per_wg consecutive
// KV heads, group of <= 16 query heads, split s).  Its 4 waves are spread
// over the KV heads: with 4 heads per workgroup each wave takes one head and
// all of the split's tiles (the 4 waves read adjacent slots of the same token
// rows, so cache lines are shared inside the CU); with fewer heads per
// workgroup the waves of one head take its tiles round-robin and merge their
// partial softmax states in LDS at the end.
template <int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void tq_decode_stage1_kernel(DecodeArgs a) {
  using T = Preset<P>;
  constexpr int kMergeStride = kD + 4;  // merge rows: 16-byte aligned, banks rotate per head
  // fp32 query scratch (up to 64 rows), later reused as the merge area
  __shared__ __attribute__((aligned(16))) float smem[kWaves * 16 * kMergeStride + 2 * kWaves * 16];
  __shared__ __attribute__((aligned(16))) _Float16 qh[kWaves * 16][kD + 8];
  float(*qf)[kD] = reinterpret_cast<float(*)[kD]>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.num_splits, Hk = a.num_kv_heads, Hq = a.num_q_heads, g = a.group;
  const int HW = a.heads_per_wg;  // 1, 2 or 4
  const int wph = kWaves / HW;    // waves per KV head
  int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int hgrp = lg % (Hk / HW);  // fastest: neighbouring heads share cache lines
  lg /= Hk / HW;
  const int hg = lg % a.head_groups;
  lg /= a.head_groups;
  const int s = lg % S;
  const int b = lg / S;
  const int hs = wave / wph;  // this wave's head slot in the workgroup
  const int phase = wave % wph;
  const int hk = hgrp * HW + hs;

  const int seqlen = a.seq_lens[b];
  const int ntiles = (seqlen + 15) >> 4;
  const int tps = (ntiles + S - 1) / S;
  const int t_begin = s * tps;
  const int t_end = min(t_begin + tps, ntiles);
  const int h0 = hg * 16;
  const int geff = min(16, g - h0);
  // partial row of query head h0 + j of KV head hgrp*HW + k
  auto part_row = [&](int k, int j) {
    return a.partials + ((static_cast<int64_t>(b) * Hq + (hgrp * HW + k) * g + h0 + j) * S + s) * (kD + 1);
  };

  if (t_begin >= t_end) {  // empty split: zero partial, lse = -inf
    for (int idx = tid; idx < HW * geff * (kD + 1); idx += kThreads) {
      const int k = idx / (geff * (kD + 1)), r = idx % (geff * (kD + 1));
      const int j = r / (kD + 1), d = r % (kD + 1);
      part_row(k, j)[d] = d == kD ? -INFINITY : 0.f;
    }
    return;
  }

  // ---- first tile's loads go out before the query prologue ----
  const int hl = lane & 15, q4 = lane >> 4;
  const int bs_log2 = 31 - __clz(a.block_size);
  const int64_t blk_bytes = static_cast<int64_t>(a.block_size) * Hk * T::kSlot;
  const uint32_t row = static_cast<uint32_t>(Hk * T::kSlot);
  const int32_t* btab = a.block_table + static_cast<int64_t>(b) * a.bt_stride;
  const LaneOff<P> off = lane_offsets<P>(hl, q4, hk, Hk);
  const int t_first = t_begin + __builtin_amdgcn_readfirstlane(phase);
  auto tile_base = [&](int t) -> const uint8_t* {
    const int tok0 = t * 16;
    const int blk = __builtin_amdgcn_readfirstlane(btab[tok0 >> bs_log2]);
    return a.cache + static_cast<int64_t>(blk) * blk_bytes + static_cast<int64_t>(tok0 & (a.block_size - 1)) * row;
  };
  TileRegs<P> ra, rb;
  if (t_first < t_end) load_tile<P>(tile_base(t_first), row, off, ra);

  // ---- query rows of the workgroup's heads: sign flip + Walsh-Hadamard
  // (MSE keys), scale by softmax scale * log2(e), fp16 in MFMA operand order
  const int nrows = HW * 16;
  const bool qbf16 = a.q_bf16 != 0;
  for (int idx = tid; idx < nrows * kD; idx += kThreads) {
    const int r = idx >> 7, d = idx & (kD - 1);
    const int k = r >> 4, j = r & 15;
    float v = 0.f;
    if (j < geff) v = widen16(a.query[(static_cast<int64_t>(b) * Hq + (hgrp * HW + k) * g + h0 + j) * kD + d], qbf16);
    if (!T::kFp8) v *= a.signs[d];
    qf[r][d] = v;
  }
  __syncthreads();
  if (!T::kFp8) {
    for (int hsz = 1; hsz < kD; hsz <<= 1) {
      for (int pi = tid; pi < nrows * (kD / 2); pi += kThreads) {
        const int r = pi / (kD / 2), k = pi % (kD / 2);
        const int i0 = (k / hsz) * 2 * hsz + (k % hsz), i1 = i0 + hsz;
        const float x0 = qf[r][i0], x1 = qf[r][i1];
        qf[r][i0] = x0 + x1;
        qf[r][i1] = x0 - x1;
      }
      __syncthreads();
    }
  }
  const float qs = T::kFp8 ? a.qscale : a.qscale * 0.08838834764831845f;  // 1/sqrt(128) of the rotation
  for (int idx = tid; idx < nrows * kD; idx += kThreads) {
    const int r = idx >> 7, d = idx & (kD - 1);
    qh[r][qh_pos<P>(d)] = static_cast<_Float16>(qf[r][d] * qs);
  }

  // codebook byte tables (fp16 centroids split into low / high bytes)
  tq::Lut8 la{}, lb{};
  if (!T::kFp8) {
    uint32_t hb[16];
#pragma unroll
    for (int i = 0; i < (1 << (T::kFp8 ? 0 : T::kKb)); ++i)
      hb[i] = __half_as_ushort(__float2half_rn(a.centroids[i]));
    auto pack = [&](int base, int shift) {
      return ((hb[base] >> shift) & 0xFF) | (((hb[base + 1] >> shift) & 0xFF) << 8) |
             (((hb[base + 2] >> shift) & 0xFF) << 16) | (((hb[base + 3] >> shift) & 0xFF) << 24);
    };
    la = {pack(0, 0), pack(4, 0), pack(0, 8), pack(4, 8)};
    if (T::kKb == 4) lb = {pack(8, 0), pack(12, 0), pack(8, 8), pack(12, 8)};
  }
  __syncthreads();

  half8 bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = *reinterpret_cast<const half8*>(&qh[hs * 16 + hl][q4 * 32 + c * 8]);

  // ---- main loop over this wave's tiles, next tile's loads in flight ----
  Softmax sm{-INFINITY, 0.f, 0.f};
  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The prefetch is unconditional (past the wave's last tile it re-reads
  // that tile, an L2 hit) so that every path into the loop has the same loads
  // in flight and the waits stay exact; the scheduling barriers keep each
  // prefetch issued before the compute of the current tile.
  const int stride = __builtin_amdgcn_readfirstlane(wph);
  int t = t_first;
  while (t < t_end) {
    load_tile<P>(tile_base(min(t + stride, t_end - 1)), row, off, rb);
    __builtin_amdgcn_sched_barrier(0);
    tile_step<P>(ra, off, row, la, lb, bq, min(16, seqlen - t * 16), sm, acc);
    t += stride;
    if (t >= t_end) break;
    load_tile<P>(tile_base(min(t + stride, t_end - 1)), row, off, ra);
    __builtin_amdgcn_sched_barrier(0);
    tile_step<P>(rb, off, row, la, lb, bq, min(16, seqlen - t * 16), sm, acc);
    t += stride;
  }
  float m_run = sm.m, l_run = sm.l, z_run = sm.z;

  // ---- per-wave totals: lane quarters hold disjoint tokens ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  z_run += __shfl_xor(z_run, 16, 64);
  z_run += __shfl_xor(z_run, 32, 64);
  // unnormalized output of query head hl, dims 32*q4 + 8*i + n
  float o[4][8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int pos = T::kVb == 4 ? tq::val4_pos(n) : tq::val3_pos(n);
    const float unscale = static_cast<float>(1u << (24 - pos));
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i][n] = fmaf(acc[n][i], unscale, z_run);
  }

  // ---- merge the waves of each head in LDS (reusing the query scratch) ----
  // Each wave scales its unnormalized output by 2^(m_w - M) / l (M: max over
  // the head's waves, l: merged softmax sum) and writes it as
  // [wave][query head][dim]; the workgroup sums the waves of each head and
  // writes every partial row with consecutive lanes on consecutive dims.
  __syncthreads();
  float* mo = smem;                               // [wave][16][kMergeStride]
  float* mm = smem + kWaves * 16 * kMergeStride;  // [wave][16] maxima
  float* ml = mm + kWaves * 16;                   // [wave][16] sums
  if (q4 == 0) {
    mm[wave * 16 + hl] = m_run;
    ml[wave * 16 + hl] = l_run;
  }
  __syncthreads();
  auto head_stats = [&](int hslot, int j, float& M, float& lsum) {
    M = -INFINITY;
    for (int k = 0; k < wph; ++k) M = fmaxf(M, mm[(hslot * wph + k) * 16 + j]);
    lsum = 0.f;
    for (int k = 0; k < wph; ++k) {
      const float mw = mm[(hslot * wph + k) * 16 + j];
      lsum = fmaf(mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M), ml[(hslot * wph + k) * 16 + j], lsum);
    }
  };
  {
    float M, lsum;
    head_stats(hs, hl, M, lsum);
    const float f = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    const float sc = lsum > 0.f ? f / lsum : 0.f;
    float* rowp = mo + (wave * 16 + hl) * kMergeStride + 32 * q4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 lo = {o[i][0] * sc, o[i][1] * sc, o[i][2] * sc, o[i][3] * sc};
      f32x4 hi = {o[i][4] * sc, o[i][5] * sc, o[i][6] * sc, o[i][7] * sc};
      *reinterpret_cast<f32x4*>(rowp + 8 * i) = lo;
      *reinterpret_cast<f32x4*>(rowp + 8 * i + 4) = hi;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < HW * geff * kD; idx += kThreads) {
    const int k = idx / (geff * kD), r = idx % (geff * kD);
    const int j = r >> 7, d = r & (kD - 1);
    float v = 0.f;
    for (int w = 0; w < wph; ++w) v += mo[((k * wph + w) * 16 + j) * kMergeStride + d];
    part_row(k, j)[d] = v;
  }
  if (tid < HW * geff) {
    const int k = tid / geff, j = tid % geff;
    float M, lsum;
    head_stats(k, j, M, lsum);
    part_row(k, j)[kD] = (M + log2f(lsum)) * kLn2;
  }
}

// ---------------------------------------------------------------- stage 2

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__global__ __launch_bounds__(256) void tq_decode_stage2_kernel(const float* __restrict__ partials, int rows, int S,
                                                               void* out, int out_dtype, float* lse_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* base = partials + static_cast<int64_t>(row) * S * (kD + 1);
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, base[static_cast<int64_t>(s) * (kD + 1) + kD]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float o0 = 0.f, o1 = 0.f, den = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float* ps = base + static_cast<int64_t>(s) * (kD + 1);
      const float ls = ps[kD];
      const float w = ls == -INFINITY ? 0.f : expf(ls - M);
      den += w;
      o0 = fmaf(w, ps[lane], o0);
      o1 = fmaf(w, ps[lane + 64], o1);
    }
    o0 /= den;
    o1 /= den;
    lse = M + logf(den);
  }
  const int64_t ob = static_cast<int64_t>(row) * kD;
  if (out_dtype == TQ_F32) {
    static_cast<float*>(out)[ob + lane] = o0;
    static_cast<float*>(out)[ob + lane + 64] = o1;
  } else if (out_dtype == TQ_F16) {
    static_cast<__half*>(out)[ob + lane] = __float2half_rn(o0);
    static_cast<__half*>(out)[ob + lane + 64] = __float2half_rn(o1);
  } else {
    static_cast<uint16_t*>(out)[ob + lane] = f32_to_bf16_rne(o0);
    static_cast<uint16_t*>(out)[ob + lane + 64] = f32_to_bf16_rne(o1);
  }
  if (lse_out && lane == 0) lse_out[row] = lse;
}

template <int P>
int launch_stage1(const DecodeArgs& a, int64_t nblocks, hipStream_t stream) {
  hipLaunchKernelGGL(tq_decode_stage1_kernel<P>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int stage1(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
           int32_t num_kv_heads, const void* kv_cache, int32_t block_size, const int32_t* block_table,
           int32_t block_table_stride, const int32_t* seq_lens, const float* signs, const float* centroids,
           float scale, int32_t num_kv_splits, void* workspace, hipStream_t stream) {
  DecodeArgs a;
  a.query = static_cast<const uint16_t*>(query);
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.signs = signs;
  a.centroids = centroids;
  a.partials = static_cast<float*>(workspace);
  a.qscale = scale * kLog2e;
  a.q_bf16 = q_dtype == TQ_BF16;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_groups = (a.group + 15) / 16;
  a.block_size = block_size;
  a.bt_stride = block_table_stride;
  a.num_splits = num_kv_splits;
  // Heads per workgroup: 4 when there are enough (sequence, split, head
  // group) units to keep ~3 workgroups on each of the 256 CUs, else fewer
  // (the waves of one head then share its tiles).
  const int64_t units = static_cast<int64_t>(batch) * a.head_groups * num_kv_splits;
  a.heads_per_wg = 1;
  for (int hw : {4, 2}) {
    if (num_kv_heads % hw == 0 && units * (num_kv_heads / hw) >= 768) {
      a.heads_per_wg = hw;
      break;
    }
  }
  const int64_t nblocks = units * (num_kv_heads / a.heads_per_wg);
  if (nblocks > 0x7FFFFFFF) return TQ_EUNSUPPORTED;
  switch (layout->preset) {
    case TQ_K8V4: return launch_stage1<TQ_K8V4>(a, nblocks, stream);
    case TQ_4BIT_NC: return launch_stage1<TQ_4BIT_NC>(a, nblocks, stream);
    case TQ_K3V4_NC: return launch_stage1<TQ_K3V4_NC>(a, nblocks, stream);
    case TQ_3BIT_NC: return launch_stage1<TQ_3BIT_NC>(a, nblocks, stream);
  }
  return TQ_EPRESET;
}

int stage2(int32_t batch, int32_t num_q_heads, int32_t num_kv_splits, const void* workspace, void* out,
           int32_t out_dtype, float* lse_out, hipStream_t stream) {
  const int rows = batch * num_q_heads;
  hipLaunchKernelGGL(tq_decode_stage2_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream,
                     static_cast<const float*>(workspace), rows, num_kv_splits, out, out_dtype, lse_out);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace

extern "C" int tq_decode_stage1(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks,
                                int32_t block_size, const int32_t* block_table, int32_t block_table_stride,
                                const int32_t* seq_lens, const float* signs, const float* centroids, float scale,
                                int32_t num_kv_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int st = tq::validate_decode(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                               block_size, block_table, block_table_stride, seq_lens, signs, centroids,
                               num_kv_splits, workspace, workspace_bytes);
  if (st != TQ_OK || batch == 0) return st;
  return stage1(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, block_size, block_table,
                block_table_stride, seq_lens, signs, centroids, scale, num_kv_splits, workspace,
                static_cast<hipStream_t>(stream));
}

extern "C" int tq_decode_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                                const void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                                float* lse_out, void* stream) {
  int st = tq::validate_stage2(batch, num_q_heads, head_dim, num_kv_splits, workspace, workspace_bytes, out,
                               out_dtype);
  if (st != TQ_OK || batch == 0) return st;
  return stage2(batch, num_q_heads, num_kv_splits, workspace, out, out_dtype, lse_out,
                static_cast<hipStream_t>(stream));
}

extern "C" int tq_decode_attention(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache,
                                   int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                                   int32_t block_table_stride, const int32_t* seq_lens, const float* signs,
                                   const float* centroids, float scale, int32_t num_kv_splits, void* workspace,
                                   size_t workspace_bytes, void* out, int32_t out_dtype, float* lse_out,
                                   void* stream) {
  int st = tq_decode_validate(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                              block_size, block_table, block_table_stride, seq_lens, signs, centroids, num_kv_splits,
                              workspace, workspace_bytes, out, out_dtype);
  if (st != TQ_OK || batch == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = stage1(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, block_size, block_table,
              block_table_stride, seq_lens, signs, centroids, scale, num_kv_splits, workspace, s);
  if (st != TQ_OK) return st;
  return stage2(batch, num_q_heads, num_kv_splits, workspace, out, out_dtype, lse_out, s);
}
