// tq_decode_attention: split-KV decode attention over the compressed paged
// cache ([PR] "实现拆解" item 4: stage 1 scores and accumulates values per
// split, stage 2 merges the splits with a log-sum-exp reduction; [API]
// _decode_attention).
//
// Stage 1 work unit: one workgroup per (length-balanced tile range of one
// sequence, group of G KV heads, up to 16 query heads per KV head); its
// G * P wave64s take the range's 16-token tiles (P phases per head) and merge
// in LDS at the end.  Per tile a wave:
//   - builds the key tile (16 tokens x 128 dims) as fp16 MFMA operands: FP8
//     keys by the hardware FP8->fp16 convert, 3-bit Lloyd-Max codes two dims
//     at a time through an LDS table of fp16 centroid pairs, 2- and 4-bit
//     codes through a v_perm byte lookup of the fp16 codebook;
//   - scores S^T = K . Q^T with 4 MFMA 16x16x32 f16 (tokens on rows, query
//     heads on columns), the query rotated by the same transform (MSE
//     presets, [API] _decode_attention) and pre-scaled by scale*log2(e) and
//     a per-head power of two that keeps its fp16 operand in range;
//   - applies the per-token key norm, an online softmax in base 2, and
//   - accumulates O^T = V^T . P^T with 8 MFMA 16x16x32 f16 per pair of
//     tiles, uniform value codes entering as fp16 subnormals (no conversion)
//     with the per-token value scale folded into P and the zero point
//     accumulated on the VALU as sum(p * zero); Lloyd-Max value codes through
//     a byte lookup of their fp16 codebook.
// The GQA group rides on the MFMA's 16 columns, so the key/value bytes of a
// (token, KV head) are read and decoded once for all its query heads.
// Both block conventions of the cache (combined slots, SoA data + metadata
// regions) are read; the convention is a template parameter.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "tq.h"
#include "tq_bits.h"
#include "tq_internal.h"
#include "tq_wave.h"

namespace {

constexpr int kD = 128;  // dims of one head half: the kernels' lane layouts cover 128 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Preset code flag: head_dim 256, held as two 128-dim halves.  The packed
// key bits and value codes of a row are positional (dim i at bits B*i), so
// half h of a 256-dim slot's key data and value data is the bytes a 128-dim
// slot would hold for those 128 dims, at offset h * (bytes of a half).
constexpr int kHead256 = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef const __attribute__((address_space(4))) int32_t cint32;  // constant (scalar-loadable) memory
typedef const __attribute__((address_space(4))) float cfloat;

// Slot geometry per preset at head_dim 128 (see tq_layout_init).
template <int P>
struct Base;
template <>
struct Base<TQ_K8V4> {
  static constexpr int kFp8 = 1, kKb = 8, kVb = 4, kKdata = 128, kKps = 128, kVdata = 64, kSlot = 196, kVlm = 0;
};
template <>
struct Base<TQ_4BIT_NC> {
  static constexpr int kFp8 = 0, kKb = 4, kVb = 4, kKdata = 64, kKps = 66, kVdata = 64, kSlot = 134, kVlm = 0;
};
template <>
struct Base<TQ_K3V4_NC> {
  static constexpr int kFp8 = 0, kKb = 3, kVb = 4, kKdata = 48, kKps = 50, kVdata = 64, kSlot = 118, kVlm = 0;
};
template <>
struct Base<TQ_3BIT_NC> {
  static constexpr int kFp8 = 0, kKb = 3, kVb = 3, kKdata = 48, kKps = 50, kVdata = 48, kSlot = 102, kVlm = 0;
};
template <>
struct Base<TQ_K8V3> {
  static constexpr int kFp8 = 1, kKb = 8, kVb = 3, kKdata = 128, kKps = 128, kVdata = 48, kSlot = 180, kVlm = 0;
};
template <>
struct Base<TQ_K4V3_NC> {
  static constexpr int kFp8 = 0, kKb = 4, kVb = 3, kKdata = 64, kKps = 66, kVdata = 48, kSlot = 118, kVlm = 0;
};
template <>
struct Base<TQ_2BIT_NC> {
  static constexpr int kFp8 = 0, kKb = 2, kVb = 2, kKdata = 32, kKps = 34, kVdata = 32, kSlot = 70, kVlm = 0;
};
// Lloyd-Max values: value region [codes | fp16 norm]
template <>
struct Base<TQ_K8V3LM> {
  static constexpr int kFp8 = 1, kKb = 8, kVb = 3, kKdata = 128, kKps = 128, kVdata = 48, kSlot = 178, kVlm = 1;
};
template <>
struct Base<TQ_3BIT_LM> {
  static constexpr int kFp8 = 0, kKb = 3, kVb = 3, kKdata = 48, kKps = 50, kVdata = 48, kSlot = 100, kVlm = 1;
};
template <>
struct Base<TQ_K8V4LM> {
  static constexpr int kFp8 = 1, kKb = 8, kVb = 4, kKdata = 128, kKps = 128, kVdata = 64, kSlot = 194, kVlm = 1;
};
template <>
struct Base<TQ_4BIT_LM> {
  static constexpr int kFp8 = 0, kKb = 4, kVb = 4, kKdata = 64, kKps = 66, kVdata = 64, kSlot = 132, kVlm = 1;
};
template <>
struct Base<TQ_2BIT_LM> {
  static constexpr int kFp8 = 0, kKb = 2, kVb = 2, kKdata = 32, kKps = 34, kVdata = 32, kSlot = 68, kVlm = 1;
};

// The geometry at the head_dim of preset code PD (a preset, plus kHead256
// for two halves): fields of the whole slot; kHk / kHv are the key / value
// data bytes of one 128-dim half.
template <int PD>
struct Preset : Base<PD & 0xFF> {
  using B = Base<PD & 0xFF>;
  static constexpr int kNh = (PD & kHead256) ? 2 : 1;  // 128-dim halves
  static constexpr int kDim = 128 * kNh;
  static constexpr int kHk = B::kKdata, kHv = B::kVdata;
  static constexpr int kKdata = kNh * B::kKdata;
  static constexpr int kKps = B::kFp8 ? kKdata : kKdata + 2;
  static constexpr int kVdata = kNh * B::kVdata;
  static constexpr int kSlot = ((kKps + kVdata + (B::kVlm ? 2 : 4) + 1) / 2) * 2;
  static constexpr int kRow = kDim + static_cast<int>(tq::kPartPad);  // floats per partial row
};

// SoA convention: data row = key data + value data; metadata record = kNf
// 16-bit fields (norm, scale, zero; FP8 keys: scale, zero).
template <int P>
struct Soa {
  static constexpr int kDb = Preset<P>::kKdata + Preset<P>::kVdata;
  static constexpr int kNf = (Preset<P>::kFp8 ? 0 : 1) + (Preset<P>::kVlm ? 1 : 2);
  static constexpr int kMb = 2 * kNf;
  static_assert(kDb % 16 == 0, "SoA data rows are 16-byte multiples");
};

// The constants above follow the slot layout of tq_layout_init at head_dim 128.
template <int P>
constexpr bool preset_geometry_ok() {
  using T = Base<P>;
  return T::kKdata == (T::kFp8 ? kD : kD * T::kKb / 8) && T::kKps == (T::kFp8 ? kD : T::kKdata + 2) &&
         T::kVdata == kD * T::kVb / 8 && T::kSlot == ((T::kKps + T::kVdata + (T::kVlm ? 2 : 4) + 1) / 2) * 2;
}
static_assert(preset_geometry_ok<TQ_K8V4>() && preset_geometry_ok<TQ_4BIT_NC>() &&
                  preset_geometry_ok<TQ_K3V4_NC>() && preset_geometry_ok<TQ_3BIT_NC>() &&
                  preset_geometry_ok<TQ_K8V3>() && preset_geometry_ok<TQ_K4V3_NC>() &&
                  preset_geometry_ok<TQ_2BIT_NC>() && preset_geometry_ok<TQ_K8V3LM>() &&
                  preset_geometry_ok<TQ_3BIT_LM>() && preset_geometry_ok<TQ_K8V4LM>() &&
                  preset_geometry_ok<TQ_4BIT_LM>() && preset_geometry_ok<TQ_2BIT_LM>(),
              "slot geometry");

struct DecodeArgs {
  const uint16_t* query;
  const uint8_t* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* signs;
  const float* centroids;
  int32_t* table;   // [B][2]: first unit, number of units of each sequence
  float* part;      // [U][Hq][kRow]: normalized partial output, then natural-log LSE
  float qscale;     // softmax scale * log2(e)
  int32_t q_bf16;
  int32_t num_q_heads, num_kv_heads, group, head_groups;
  int32_t G;           // KV heads per workgroup
  int32_t P;           // waves per KV head (tile phases)
  int32_t ring_depth;  // super-tiles (P tiles each) in the LDS ring
  int32_t spt;         // 1 KB direct-to-LDS slots per tile image
  int32_t contiguous;  // G == Hk: a tile of the group is one run of 16 token rows
  int32_t dslots;      // SoA: slots of the data part of a tile image (the metadata part follows)
  int32_t soa_pad;     // SoA: pad bytes after each image row of data (a multiple of 16)
  int32_t block_size, bt_stride;
  int32_t batch, num_units;  // B, U
  int32_t window;            // sliding window in tokens, 0 = the whole sequence
};

__device__ __forceinline__ float widen16(uint32_t bits, bool bf16) {
  if (bf16) return __uint_as_float(bits << 16);
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

// x * (fp16 in the low / high half of w), rounded once to fp32.  Written as an
// fma with a +0 addend (equal to the product but for the sign of a zero
// product) so that it becomes one v_fma_mix_f32 reading the half in place
// instead of a conversion and a multiply.
__device__ __forceinline__ float mul_lo16(float x, uint32_t w) {
  return fmaf(x, static_cast<float>(__builtin_bit_cast(half2v, w)[0]), 0.0f);
}
__device__ __forceinline__ float mul_hi16(float x, uint32_t w) {
  return fmaf(x, static_cast<float>(__builtin_bit_cast(half2v, w)[1]), 0.0f);
}
// x * (high half of w) + y, rounded once.
__device__ __forceinline__ float fma_hi16(float x, uint32_t w, float y) {
  return fmaf(x, static_cast<float>(__builtin_bit_cast(half2v, w)[1]), y);
}

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs; remap
// so that consecutive *logical* ids (the KV heads of one sequence/split,
// which share cache lines) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, loc = bid / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + loc;
}

// Dword at a 2-byte aligned LDS address as two 16-bit reads joined by one
// shift-or.  A dword read there would be unaligned (several times slower on
// this LDS), and two dwords read as one pair take 8-bit offsets, too short
// for a ring entry's, so every such read would need an address add.  The
// upper half is read non-temporally only so that the compiler does not fuse
// the two halves into one unaligned dword read (LDS has no such hint).
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ uint32_t ld32_even(const uint8_t* p) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));  // LDS offset of p
  const uint16_t lo = *reinterpret_cast<lds_cu16*>(static_cast<size_t>(a));
  const uint16_t hi = __builtin_nontemporal_load(reinterpret_cast<lds_u16*>(static_cast<size_t>(a + 2)));
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// The value-code word (4 bytes; 3-bit codes use the low 3) of a lane at byte
// vo of the tile image tb.  Tile bases are 32-byte aligned and slots, key
// parts and 4- or 2-bit words even, so vo is even there (2 mod 4 for half
// the heads when the slot is 2 mod 4); 3-bit words start at 3 x the lane's
// row and may sit at any byte: an aligned pair of dwords, realigned.
template <int P>
__device__ __forceinline__ uint32_t value_word(const uint8_t* tb, uint32_t vo) {
  using T = Preset<P>;
  if constexpr (T::kSlot % 4 == 0 && T::kKps % 4 == 0 && T::kVb == 4) {
    return *reinterpret_cast<const uint32_t*>(tb + vo);
  } else if constexpr (T::kVb != 3) {
    return ld32_even(tb + vo);
  } else {
    const u32x2a4 w = *reinterpret_cast<const u32x2a4*>(tb + (vo & ~3u));
    return tq::alignbyte(w.y, w.x, vo & 3u);
  }
}

__device__ __forceinline__ uint32_t ld16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4a4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half4 as_half4(uint32_t a, uint32_t b) {
  u32x2a4 v = {a, b};
  return __builtin_bit_cast(half4, v);
}
__device__ __forceinline__ uint32_t h2_bits(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Reductions over the four lane quarters (lanes l, l^16, l^32, l^48) with
// the row-swap permutes: permlane16_swap leaves each lane holding its own
// value and that of lane l^16 (one in each result), permlane32_swap the same
// for l^32.  No LDS round trip.
__device__ __forceinline__ float quarter_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float quarter_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Byte offsets (lane constants) of what one lane reads from a tile image in
// LDS.  The image keeps every slot at the same alignment mod 16 as in the
// cache, and that alignment depends only on the token row and the head, so
// each address's alignment is a lane constant: unaligned fields are read as
// aligned dwords and realigned.
template <int P>
struct LaneOff {
  uint32_t k, ksh;  // aligned-down key chunk start, its misalignment (0 for SoA)
  uint32_t mo[4];   // slot start of token 4q + i (SoA: mo[0] = data row of token 4q)
  uint32_t vcol;    // byte offset of the lane's value-code column inside a slot / data row
  uint32_t mm0;     // SoA: metadata record of token 4q
  uint32_t sd, sm;  // SoA: image bytes between consecutive tokens' data rows / records (uniform)
};

template <int P, int SOA>
__device__ __forceinline__ uint32_t data_row(const LaneOff<P>& o, int i) {
  return SOA ? o.mo[0] + static_cast<uint32_t>(i) * o.sd : o.mo[i];
}
template <int P>
__device__ __forceinline__ uint32_t meta_rec(const LaneOff<P>& o, int i) {
  return o.mm0 + static_cast<uint32_t>(i) * o.sm;
}

// Registers one tile's loads land in.
template <int P>
struct TileRegs {
  uint32_t k[Preset<P>::kNh][8];     // per head half
  uint32_t v[Preset<P>::kNh][4];     // value words, per head half
  uint32_t sz[4];  // fp16 scale | fp16 zero << 16
  uint32_t gm[4];  // fp16 key norm (MSE keys)
};

// Where the workgroup's rows sit in the cache and how its tile image is
// laid out (see the staging notes below).
struct ImageGeom {
  uint32_t base;  // hgp * G * slot: byte offset of the group's piece in a cache row
  uint32_t row;   // Hk * slot: bytes of a cache row
  bool contiguous;
};

template <int P>
__device__ __forceinline__ void load_keys(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r);
template <int P>
__device__ __forceinline__ void load_keys_soa(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r);
template <int P>
__device__ __forceinline__ void load_token_fields_soa(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r);
template <int P>
__device__ __forceinline__ void load_value_words_soa(const uint8_t* tb, const LaneOff<P>& o,
                                                     uint32_t (&vw)[Preset<P>::kNh][4]);

// Read one tile's fields of this lane from the tile image at tb.  SoA: the
// value words arrive realigned in v[i][0].
template <int P, int SOA>
__device__ __forceinline__ void load_tile(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
  if constexpr (SOA != 0) {
    load_keys_soa<P>(tb, o, r);
    load_token_fields_soa<P>(tb, o, r);
    uint32_t vw[T::kNh][4];
    load_value_words_soa<P>(tb, o, vw);
#pragma unroll
    for (int h = 0; h < T::kNh; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[h][i] = vw[h][i];
    return;
  }
  load_keys<P>(tb, o, r);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < T::kNh; ++h)
      r.v[h][i] = value_word<P>(tb, o.mo[i] + o.vcol + static_cast<uint32_t>(h * T::kHv));
    const uint8_t* m = tb + o.mo[i];
    if constexpr (T::kSlot % 4 == 0 && (T::kKps + T::kVdata) % 4 == 0)
      r.sz[i] = *reinterpret_cast<const uint32_t*>(m + T::kKps + T::kVdata);
    else
      r.sz[i] = ld32_even(m + T::kKps + T::kVdata);  // 2 mod 4 for half the heads
    if constexpr (T::kFp8 == 0) r.gm[i] = ld16(m + T::kKdata);
  }
}

// The key words of the lane (token lane % 16, dims of its quarter), per head
// half (half h's key data starts h * kHk bytes on, a multiple of 4: both
// halves share the alignment).
template <int P>
__device__ __forceinline__ void load_keys(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
#pragma unroll
  for (int h = 0; h < T::kNh; ++h) {
    const uint8_t* kb = tb + o.k + h * T::kHk;
    uint32_t* rk = r.k[h];
    if constexpr (T::kFp8 != 0 && T::kSlot % 4 != 0) {
      // FP8 keys in slots of 2 mod 4 bytes: half the heads start 2 bytes off
      // a dword; read the aligned words around each 16-byte run and realign
      const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(kb);
      const uint32_t e0 = *reinterpret_cast<const uint32_t*>(kb + 16);
      const u32x4a4 k1 = *reinterpret_cast<const u32x4a4*>(kb + 64);
      const uint32_t e1 = *reinterpret_cast<const uint32_t*>(kb + 80);
      rk[0] = tq::alignbyte(k0.y, k0.x, o.ksh); rk[1] = tq::alignbyte(k0.z, k0.y, o.ksh);
      rk[2] = tq::alignbyte(k0.w, k0.z, o.ksh); rk[3] = tq::alignbyte(e0, k0.w, o.ksh);
      rk[4] = tq::alignbyte(k1.y, k1.x, o.ksh); rk[5] = tq::alignbyte(k1.z, k1.y, o.ksh);
      rk[6] = tq::alignbyte(k1.w, k1.z, o.ksh); rk[7] = tq::alignbyte(e1, k1.w, o.ksh);
    } else if constexpr (T::kFp8 != 0) {
      const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(kb);
      const u32x4a4 k1 = *reinterpret_cast<const u32x4a4*>(kb + 64);
      rk[0] = k0.x; rk[1] = k0.y; rk[2] = k0.z; rk[3] = k0.w;
      rk[4] = k1.x; rk[5] = k1.y; rk[6] = k1.z; rk[7] = k1.w;
    } else {
      const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(kb);
      rk[0] = k0.x; rk[1] = k0.y; rk[2] = k0.z; rk[3] = k0.w;
      if (T::kKb == 4) rk[4] = *reinterpret_cast<const uint32_t*>(kb + 16);
    }
  }
}

// The per-token fields of the lane's 4 tokens (4q .. 4q+3): value scale and
// zero, and the key norm (MSE keys).
template <int P>
__device__ __forceinline__ void load_token_fields(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* m = tb + o.mo[i];
    if constexpr (T::kSlot % 4 == 0 && (T::kKps + T::kVdata) % 4 == 0) {
      r.sz[i] = *reinterpret_cast<const uint32_t*>(m + T::kKps + T::kVdata);
    } else {
      r.sz[i] = ld32_even(m + T::kKps + T::kVdata);  // 2 mod 4 for half the heads
    }
    if constexpr (T::kFp8 == 0) r.gm[i] = ld16(m + T::kKdata);
  }
}

// The value-code words of the lane's 4 tokens (tokens 4q .. 4q+3, dims of
// lane row), realigned, straight from the tile image.
template <int P>
__device__ __forceinline__ void load_value_words(const uint8_t* tb, const LaneOff<P>& o,
                                                 uint32_t (&vw)[Preset<P>::kNh][4]) {
  using T = Preset<P>;
#pragma unroll
  for (int h = 0; h < T::kNh; ++h)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vw[h][i] = value_word<P>(tb, o.mo[i] + o.vcol + static_cast<uint32_t>(h * T::kHv));
  }
}

// SoA image: data rows are 16-byte multiples, so the key chunk and (4-bit)
// value words of a lane are 4-byte aligned; 3-bit value words and the MSE
// scale/zero pair (after the 16-bit norm) are realigned.
template <int P>
__device__ __forceinline__ void load_keys_soa(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
#pragma unroll
  for (int h = 0; h < T::kNh; ++h) {
    const uint8_t* kb = tb + o.k + h * T::kHk;
    const u32x4a4 k0 = *reinterpret_cast<const u32x4a4*>(kb);
    r.k[h][0] = k0.x; r.k[h][1] = k0.y; r.k[h][2] = k0.z; r.k[h][3] = k0.w;
    if constexpr (T::kFp8 != 0) {
      const u32x4a4 k1 = *reinterpret_cast<const u32x4a4*>(kb + 64);
      r.k[h][4] = k1.x; r.k[h][5] = k1.y; r.k[h][6] = k1.z; r.k[h][7] = k1.w;
    }
  }
}

template <int P>
__device__ __forceinline__ void load_token_fields_soa(const uint8_t* tb, const LaneOff<P>& o, TileRegs<P>& r) {
  using T = Preset<P>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t rec = meta_rec(o, i);
    if constexpr (T::kVlm != 0 && T::kFp8 != 0) {
      r.sz[i] = ld16(tb + rec);  // records of one 16-bit field: the value norm
    } else if constexpr (T::kVlm != 0) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(tb + rec);  // key norm | value norm: aligned
      r.gm[i] = w;
      r.sz[i] = w >> 16;
    } else if constexpr (T::kFp8 != 0) {
      r.sz[i] = *reinterpret_cast<const uint32_t*>(tb + rec);  // records of 4 bytes: aligned
    } else {
      r.gm[i] = ld16(tb + rec);
      const uint32_t so = rec + 2u;
      const u32x2a4 w = *reinterpret_cast<const u32x2a4*>(tb + (so & ~3u));
      r.sz[i] = tq::alignbyte(w.y, w.x, so & 3u);
    }
  }
}

template <int P>
__device__ __forceinline__ void load_value_words_soa(const uint8_t* tb, const LaneOff<P>& o,
                                                     uint32_t (&vw)[Preset<P>::kNh][4]) {
  using T = Preset<P>;
#pragma unroll
  for (int h = 0; h < T::kNh; ++h)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t vo = data_row<P, 1>(o, i) + o.vcol + static_cast<uint32_t>(h * T::kHv);
    if constexpr (T::kVb == 4) {
      vw[h][i] = *reinterpret_cast<const uint32_t*>(tb + vo);
    } else {
      const u32x2a4 w = *reinterpret_cast<const u32x2a4*>(tb + (vo & ~3u));
      vw[h][i] = tq::alignbyte(w.y, w.x, vo & 3u);
    }
  }
}

static_assert(tq::kKey3LutCopies == 64, "pair table: 256-byte entries (one dword per lane copy)");

// Dword at LDS byte address `addr`.
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;
__device__ __forceinline__ uint32_t lds_u32(uint32_t addr) {
  return *reinterpret_cast<lds_cu32*>(static_cast<size_t>(addr));
}

// (x & mask) | y in one v_and_or_b32.  The compiler turns an or of disjoint
// bits into an add, which it then cannot fuse with the and.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t y) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(y));
  return r;
}

// Key tile operand for one lane (token = lane % 16, its 32 dims of quarter q
// in head half hh).  SOA: the key words are aligned (sh unused).  klane: LDS
// address of the lane's copy of the 3-bit pair table's entry 0 (entry f at
// klane + 256 f); the table starts at LDS address 0, so klane's bits 8..13
// are clear and an or places the entry.
template <int P, int SOA>
__device__ __forceinline__ void key_operand(const TileRegs<P>& rr, int hh, uint32_t sh, const tq::Lut8& la,
                                            const tq::Lut8& lb, uint32_t klane, half8 A[4]) {
  using T = Preset<P>;
  const uint32_t* k = rr.k[hh];
  if constexpr (T::kFp8 != 0) {
    uint32_t hv[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hv[2 * i] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[i], 1.0f, false));
      hv[2 * i + 1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[i], 1.0f, true));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) A[c] = as_half8(hv[4 * c], hv[4 * c + 1], hv[4 * c + 2], hv[4 * c + 3]);
  } else if constexpr (T::kKb == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = SOA ? k[c] : tq::alignbyte(k[c + 1], k[c], sh);
      uint32_t e0, e1, o0, o1;
      tq::lut16(w & 0x0F0F0F0Fu, la, lb, e0, e1);
      tq::lut16((w >> 4) & 0x0F0F0F0Fu, la, lb, o0, o1);
      A[c] = as_half8(e0, e1, o0, o1);
    }
  } else if constexpr (T::kKb == 2) {
    const uint32_t w0 = SOA ? k[0] : tq::alignbyte(k[1], k[0], sh);
    const uint32_t w1 = SOA ? k[1] : tq::alignbyte(k[2], k[1], sh);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = c < 2 ? w0 : w1;
      uint32_t a0, a1, b0, b1;
      tq::lut8(tq::key2_selector(w, 2 * (c & 1)), la, a0, a1);
      tq::lut8(tq::key2_selector(w, 2 * (c & 1) + 1), la, b0, b1);
      A[c] = as_half8(a0, a1, b0, b1);
    }
  } else {
    // 3-bit keys: 16 lookups of two dims each in the LDS pair table (a
    // field extract and an address per lookup, against ~4 VALU operations
    // per two dims through selector bytes and byte permutes)
    const uint32_t w0 = SOA ? k[0] : tq::alignbyte(k[1], k[0], sh);
    const uint32_t w1 = SOA ? k[1] : tq::alignbyte(k[2], k[1], sh);
    const uint32_t w2 = SOA ? k[2] : tq::alignbyte(k[3], k[2], sh);
    // one shift (or funnel shift) and one and-or per lookup
    uint32_t d[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = lds_u32(and_or(tq::key3_pair_window(w0, w1, w2, j), 0x3F00u, klane));
#pragma unroll
    for (int c = 0; c < 4; ++c) A[c] = as_half8(d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]);
  }
}

// Online-softmax state of one lane: query head lane % 16; the 4 lane quarters
// hold disjoint tokens and share the reference maximum m.
// The MFMA scores come out in units of the lane's query scale: s = f * s'
// with f = 2^-e chosen per query head when its fp16 operand is built, so the
// operand's largest value sits in [2^13, 2^14) whatever the query's
// magnitude (no fp16 overflow for large queries, no subnormals for small
// ones).  m is in true units; mt = (m + kLazyRescaleLog2) / f is the rescale
// threshold in the units of the raw scores.
struct Softmax {
  float m, l, z;  // reference max (log2 domain), sum of p, sum of p * zero
  float f, fi;    // the lane's score unit 2^-e and its inverse 2^e
  float mt;       // (m + kLazyRescaleLog2) * fi
  float mx;       // exact running maximum (log2 domain; kept by the sparse-V gate only)
};

// Largest growth of p = 2^(s - m) tolerated before the accumulators are
// rescaled; p * value_scale must also stay inside fp16.
constexpr float kLazyRescaleLog2 = 8.0f;

__device__ __forceinline__ void set_max(Softmax& sm, float m) {
  sm.m = m;
  sm.mt = (m + kLazyRescaleLog2) * sm.fi;
}

// A scored tile waiting for its value accumulation: value accumulation runs
// on 16x16x32 MFMAs over two tiles at once (32 tokens on the reduction
// axis), so the first tile of a pair is held here until the second is
// scored.
template <int P>
struct PendingTile {
  uint32_t vw[Preset<P>::kNh][4];  // per head half: value-code words of tokens 4q .. 4q+3 (dims of lane row)
  half4 pv;                        // p * value_scale of those tokens, fp16
};

// The opt-in sparse-V gate (gate > 0, uniform; glg = log2(gate)): a token
// whose factor exp(s - mx) against the exact running maximum mx of its head
// (over the tokens the work unit has scored so far, this tile included) is
// below the gate keeps its weight p in the softmax sum but adds no value (its
// value weight ps and its zero-point term drop).  mx never exceeds the final
// maximum, so every gated token also has exp(s - max) < gate.  Returns the
// threshold in raw score units (-inf with the gate off); lmax: the lane's
// largest raw score of the tile.
__device__ __forceinline__ float gate_threshold(float gate, float glg, float lmax, Softmax& sm) {
  if (!(gate > 0.f)) return -INFINITY;
  sm.mx = fmaxf(sm.mx, quarter_max(lmax) * sm.f);
  return (sm.mx + glg) * sm.fi;
}
__device__ __forceinline__ void sparse_v_gate(float gthr, const float sco[4], float ps[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (sco[i] < gthr) ps[i] = 0.f;
}
__device__ __forceinline__ float gated_p(float gthr, float sco, float p) { return sco < gthr ? 0.f : p; }

// Whether either tile of a pair has a value weight left (false only when the
// sparse-V gate dropped every token of both: the pair's value work is skipped).
template <int P>
__device__ __forceinline__ bool pair_has_values(const PendingTile<P>& x, const PendingTile<P>& y) {
  const u32x2a4 a = __builtin_bit_cast(u32x2a4, x.pv), b = __builtin_bit_cast(u32x2a4, y.pv);
  return __any(((a.x | a.y | b.x | b.y) & 0x7FFF7FFFu) != 0u);
}

// Score one tile and update the online softmax.  valid: tokens of the tile
// before the sequence end (1..16).  On return `cur` holds the tile's value
// words and weights; if the running maximum moved, the accumulators and the
// pending tile (when `have_pend`) are rescaled to it.  bq: 4 query operands
// per head half; acc: 8 accumulators per head half.
template <int P, int SOA>
__device__ __forceinline__ void score_tile(const TileRegs<P>& r, const LaneOff<P>& o, const tq::Lut8& la,
                                           const tq::Lut8& lb, uint32_t klane, const half8* bq, int valid,
                                           int skip, float gate,
                                           float glg, Softmax& sm, f32x4* acc, PendingTile<P>& pend,
                                           bool have_pend, PendingTile<P>& cur) {
  using T = Preset<P>;
  // two independent accumulation chains halve the dependent-MFMA latency
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < T::kNh; ++h) {
    half8 A[4];
    key_operand<P, SOA>(r, h, o.ksh, la, lb, klane, A);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], bq[4 * h], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], bq[4 * h + 1], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], bq[4 * h + 2], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], bq[4 * h + 3], s1, 0, 0, 0);
  }

  // per token: fp16 value scale (low half) and zero (high half)
  float sco[4];
  uint32_t sz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sc = s0[i] + s1[i];
    sco[i] = T::kFp8 ? sc : mul_lo16(sc, r.gm[i]);
    sz[i] = r.sz[i];
  }
  const int lane = threadIdx.x & 63;
  if (__builtin_expect(valid < 16 || skip > 0, 0)) {  // tokens past the end or before the window drop out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * (lane >> 4) + i;
      if (j >= valid || j < skip) {
        sco[i] = -INFINITY;
        sz[i] = 0u;  // the bytes past the end may hold anything (a NaN scale)
      }
    }
  }
  // The rescale test needs no cross-lane maximum: a head's maximum over its
  // four lane quarters exceeds the threshold iff one of the lanes' does.
  const float lmax = fmaxf(fmaxf(sco[0], sco[1]), fmaxf(sco[2], sco[3]));
  float p[4], ps[4], pmax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(fmaf(sco[i], sm.f, -sm.m));
    ps[i] = mul_lo16(p[i], sz[i]);
    pmax = fmaxf(pmax, ps[i]);
  }
  if (__any(lmax > sm.mt || pmax > 65504.f)) {  // rescale the accumulators (and the pending tile) to the new maximum
    const float m_cand = fmaxf(sm.m, quarter_max(lmax) * sm.f);
    const float alpha = __builtin_amdgcn_exp2f(sm.m - m_cand);
#pragma unroll
    for (int n = 0; n < 8 * T::kNh; ++n) acc[n] *= alpha;
    sm.l *= alpha;
    sm.z *= alpha;
    set_max(sm, m_cand);
    if (have_pend) {
      const _Float16 ah = static_cast<_Float16>(alpha);
      pend.pv = pend.pv * ah;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sco[i], sm.f, -sm.m));
      ps[i] = mul_lo16(p[i], sz[i]);
    }
  }
  const float gthr = gate_threshold(gate, glg, lmax, sm);
  sparse_v_gate(gthr, sco, ps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.l += p[i];
    if (!T::kVlm) sm.z = fma_hi16(gated_p(gthr, sco[i], p[i]), sz[i], sm.z);  // Lloyd-Max values have no zero point
  }
  half2v ps01 = {static_cast<_Float16>(ps[0]), static_cast<_Float16>(ps[1])};
  half2v ps23 = {static_cast<_Float16>(ps[2]), static_cast<_Float16>(ps[3])};
  cur.pv = as_half4(h2_bits(ps01), h2_bits(ps23));
#pragma unroll
  for (int h = 0; h < T::kNh; ++h)
#pragma unroll
  for (int i = 0; i < 4; ++i) cur.vw[h][i] = r.v[h][i];
}

// O^T += V^T P^T over two scored tiles, one 128-dim head half (av / bv: the
// tiles' value words of that half; bp: their weights): 8 MFMA 16x16x32 f16,
// one per block of 16 dims; reduction index k = 8q + j holds token 4q + j of tile `a`
// (j < 4) or token 4q + j - 4 of tile `b`.
// Lloyd-Max values (lv: their fp16 codebook) go through the byte-permute
// lookup instead: selector n holds code n (dim 8 * row + n) of the tile's 4
// tokens, so one lookup yields two tokens' fp16 centroids for that dim
// (4-bit codes: two 8-entry tables, picked by bit 3).
struct ValLut {
  tq::Lut8 lo, hi;  // fp16 centroids 0..7 and (4-bit codes) 8..15
};

template <int P>
__device__ __forceinline__ void accumulate_half(const uint32_t (&av)[4], const uint32_t (&bv)[4], const half8& bp,
                                                const ValLut& lv, f32x4* acc) {
  using T = Preset<P>;
  if constexpr (T::kVlm != 0) {
    uint32_t sa[8], sb[8];
    if constexpr (T::kVb == 4) {
      tq::lm4_value_selectors(av, sa);
      tq::lm4_value_selectors(bv, sb);
    } else if constexpr (T::kVb == 2) {
      tq::lm2_value_selectors(av, sa);
      tq::lm2_value_selectors(bv, sb);
    } else {
      tq::lm_value_selectors(av, sa);
      tq::lm_value_selectors(bv, sb);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      uint32_t a0, a1, b0, b1;
      if constexpr (T::kVb == 4) {
        tq::lut16(sa[n], lv.lo, lv.hi, a0, a1);
        tq::lut16(sb[n], lv.lo, lv.hi, b0, b1);
      } else {
        tq::lut8(sa[n], lv.lo, a0, a1);
        tq::lut8(sb[n], lv.lo, b0, b1);
      }
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a0, a1, b0, b1), bp, acc[n], 0, 0, 0);
    }
  } else if constexpr (T::kVb == 4) {
    const tq::Val4Pre a01 = tq::val4_pre(av[0], av[1]), a23 = tq::val4_pre(av[2], av[3]);
    const tq::Val4Pre b01 = tq::val4_pre(bv[0], bv[1]), b23 = tq::val4_pre(bv[2], bv[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          as_half8(tq::val4_get(a01, n), tq::val4_get(a23, n), tq::val4_get(b01, n), tq::val4_get(b23, n)), bp,
          acc[n], 0, 0, 0);
  } else if constexpr (T::kVb == 2) {
    const tq::Val2Pre a01 = tq::val2_pre(av[0], av[1]), a23 = tq::val2_pre(av[2], av[3]);
    const tq::Val2Pre b01 = tq::val2_pre(bv[0], bv[1]), b23 = tq::val2_pre(bv[2], bv[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          as_half8(tq::val2_get(a01, n), tq::val2_get(a23, n), tq::val2_get(b01, n), tq::val2_get(b23, n)), bp,
          acc[n], 0, 0, 0);
  } else {
    const tq::Val3Pre a01 = tq::val3_pre(av[0], av[1]), a23 = tq::val3_pre(av[2], av[3]);
    const tq::Val3Pre b01 = tq::val3_pre(bv[0], bv[1]), b23 = tq::val3_pre(bv[2], bv[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          as_half8(tq::val3_get(a01, n), tq::val3_get(a23, n), tq::val3_get(b01, n), tq::val3_get(b23, n)), bp,
          acc[n], 0, 0, 0);
  }
}

// Both head halves of a pair of scored tiles (acc: 8 accumulators per half).
template <int P>
__device__ __forceinline__ void accumulate_pair(const PendingTile<P>& a, const PendingTile<P>& b,
                                                const ValLut& lv, f32x4* acc) {
  using T = Preset<P>;
  u32x2a4 pa = __builtin_bit_cast(u32x2a4, a.pv), pb = __builtin_bit_cast(u32x2a4, b.pv);
  const half8 bp = as_half8(pa.x, pa.y, pb.x, pb.y);
#pragma unroll
  for (int h = 0; h < T::kNh; ++h) accumulate_half<P>(a.vw[h], b.vw[h], bp, lv, acc + 8 * h);
}

// Value of lane l ^ 8 (the other half of the lane's row of 16): DPP row_ror:8.
__device__ __forceinline__ float swap8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap8(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false));
}

// Two tiles of a super-tile scored as one, for GQA groups of at most 8
// query heads.  The score MFMA gives each tile a 16 x 16 block whose
// columns 8..15 carry no query head; tile B's columns 0..7 move into them
// (lanes 8..15 of each row of 16 take lane l - 8's value, one masked DPP move
// per value), so one softmax pass over 4 values per lane covers both tiles:
// lane (row r, column c) holds token 4(l/16)+i of tile A (c < 8) or of tile
// B (c >= 8) for query head c % 8.  Lanes c and c ^ 8 hold the same head and
// keep the same running maximum (their maxima are combined); each keeps the
// sums of its own tile's tokens, added together at the end.  The per-token
// key norm and value scale/zero come from the lane's own tile: one set of
// reads for both tiles.  The value MFMA then takes tile A's weights from the
// lane itself and tile B's from lane c + 8.  Columns 8..15 of the output
// accumulators hold nothing used.
template <int P, int SOA>
__device__ __forceinline__ void score_pair_packed(const uint8_t* imgA, const uint8_t* imgB, const LaneOff<P>& o,
                                                  const tq::Lut8& la, const tq::Lut8& lb, const ValLut& lv,
                                                  uint32_t klane, const half8* bq, int validA, int validB, int skipA, int skipB,
                                                  float gate, float glg, Softmax& sm, f32x4* acc) {
  using T = Preset<P>;
  static_assert(T::kNh == 1, "packed pairs: head_dim 128");
  const int lane = threadIdx.x & 63;
  const bool tileB = (lane & 8) != 0;
  TileRegs<P> rA, rB, own;
  if constexpr (SOA != 0) {
    load_keys_soa<P>(imgA, o, rA);
    load_keys_soa<P>(imgB, o, rB);
    load_token_fields_soa<P>(tileB ? imgB : imgA, o, own);
  } else {
    load_keys<P>(imgA, o, rA);
    load_keys<P>(imgB, o, rB);
    load_token_fields<P>(tileB ? imgB : imgA, o, own);
  }
  // one accumulation chain per tile: the two tiles' chains interleave
  half8 A[4];
  key_operand<P, SOA>(rA, 0, o.ksh, la, lb, klane, A);
  f32x4 sa = {0.f, 0.f, 0.f, 0.f};
  sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], bq[0], sa, 0, 0, 0);
  sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], bq[1], sa, 0, 0, 0);
  sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], bq[2], sa, 0, 0, 0);
  sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], bq[3], sa, 0, 0, 0);
  key_operand<P, SOA>(rB, 0, o.ksh, la, lb, klane, A);
  f32x4 sb = {0.f, 0.f, 0.f, 0.f};
  sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], bq[0], sb, 0, 0, 0);
  sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], bq[1], sb, 0, 0, 0);
  sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], bq[2], sb, 0, 0, 0);
  sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], bq[3], sb, 0, 0, 0);

  // per token: fp16 value scale (low half) and zero (high half)
  float sco[4];
  uint32_t sz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // lanes 8..15 of each row of 16 take tile B's value of lane l - 8
    const float sc = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(sa[i]), __float_as_int(sb[i]), 0x118, 0xF, 0xC, false));
    sco[i] = T::kFp8 ? sc : mul_lo16(sc, own.gm[i]);
    sz[i] = own.sz[i];
  }
  const int valid = tileB ? validB : validA;
  const int skip = tileB ? skipB : skipA;
  if (__builtin_expect(validA < 16 || validB < 16 || skipA > 0, 0)) {  // (a window start falls in tile A)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * (lane >> 4) + i;
      if (j >= valid || j < skip) {
        sco[i] = -INFINITY;
        sz[i] = 0u;  // the bytes past the end may hold anything (a NaN scale)
      }
    }
  }
  float lmax = fmaxf(fmaxf(sco[0], sco[1]), fmaxf(sco[2], sco[3]));
  lmax = fmaxf(lmax, swap8(lmax));  // the head's maximum over both tiles
  float p[4], ps[4], pmax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(fmaf(sco[i], sm.f, -sm.m));
    ps[i] = mul_lo16(p[i], sz[i]);
    pmax = fmaxf(pmax, ps[i]);
  }
  if (__any(lmax > sm.mt || pmax > 65504.f)) {  // rescale the accumulators to the new maximum (same on lanes c and c ^ 8)
    const float m_cand = fmaxf(sm.m, quarter_max(lmax) * sm.f);
    const float alpha = __builtin_amdgcn_exp2f(sm.m - m_cand);
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    sm.l *= alpha;
    sm.z *= alpha;
    set_max(sm, m_cand);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sco[i], sm.f, -sm.m));
      ps[i] = mul_lo16(p[i], sz[i]);
    }
  }
  const float gthr = gate_threshold(gate, glg, lmax, sm);
  sparse_v_gate(gthr, sco, ps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sm.l += p[i];
    if (!T::kVlm) sm.z = fma_hi16(gated_p(gthr, sco[i], p[i]), sz[i], sm.z);  // Lloyd-Max values have no zero point
  }
  // value weights: tile A's from this lane, tile B's from lane c + 8
  half2v ps01 = {static_cast<_Float16>(ps[0]), static_cast<_Float16>(ps[1])};
  half2v ps23 = {static_cast<_Float16>(ps[2]), static_cast<_Float16>(ps[3])};
  PendingTile<P> ta, tb;
  ta.pv = as_half4(h2_bits(ps01), h2_bits(ps23));
  tb.pv = as_half4(swap8(h2_bits(ps01)), swap8(h2_bits(ps23)));
  // every token of both tiles gated: no value reads, no value products
  if (gate > 0.f && !__any(ps[0] != 0.f || ps[1] != 0.f || ps[2] != 0.f || ps[3] != 0.f)) return;
  if constexpr (SOA != 0) {
    load_value_words_soa<P>(imgA, o, ta.vw);
    load_value_words_soa<P>(imgB, o, tb.vw);
  } else {
    load_value_words<P>(imgA, o, ta.vw);
    load_value_words<P>(imgB, o, tb.vw);
  }
  accumulate_pair<P>(ta, tb, lv, acc);
}

// ---- tile staging: cache rows -> LDS ring by direct-to-LDS loads ----
//
// A tile is 16 consecutive token rows of the cache restricted to the
// workgroup's G KV heads: 16 row pieces of G * slot bytes at a row stride of
// row = Hk * slot.  With G == Hk the pieces form one contiguous run of 16 *
// row bytes (tile bases are 32-byte aligned).  Otherwise each piece is
// fetched as the 16-byte chunks that cover it, from its start aligned down
// to 16 bytes (cpp chunks per piece), so the image keeps every byte at its
// cache alignment mod 16 and a few neighbouring bytes ride along.  Chunks go
// out in 1 KB "DMA slots" of 64 lanes x 16 bytes; a tile image takes spt
// slots (lanes past the last chunk repeat it into the image's padding).  A
// super-tile is P consecutive tiles; one ring entry holds one super-tile.
// Tile p of a super-tile is staged by the G waves of phase p (the waves
// that will compute it): wave (hh, p) issues slots hh, hh + G, ... of it,
// so a wave needs one block id and one base address per super-tile.
template <int P, int SOA>
struct Ring {
  static constexpr int kLoads = tq::max_dma_loads(P & 0xFF, SOA != 0, Preset<P>::kDim);
  uint32_t lds_base;       // LDS byte address of ring entry 0 (uniform)
  uint32_t entry;          // bytes per ring entry (P * spt KB)
  int my_loads;            // DMA slots per super-tile issued by this wave
  uint32_t dst[kLoads];    // per load: LDS offset inside the entry (uniform)
  uint32_t off[kLoads];    // per load: this lane's chunk offset from the tile base
  uint32_t meta_loads;     // SoA: bit k set when load k reads the metadata part (uniform)
};

// One direct-to-LDS load of 16 bytes per lane, non-temporal: the data is
// read once.  LDS destination = m0 + 16 * lane.  Written as inline assembly
// so that the compiler does not guard every later LDS read with a full
// vmcnt(0) wait; the ring's own waits (vm_wait + barrier) order the reads.
// m0 is a reserved register the compiler cannot be told about: the stage-1
// kernels use m0 for nothing else (checked in their ISA), so setting it here
// disturbs no compiler-managed state.
// Addressing: uniform 64-bit base in SGPRs + this lane's 32-bit byte offset.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(m0) : "memory");
}

// Wait until at most n vector-memory loads of this wave are outstanding
// (n uniform).  Loads retire in order, so every older load has completed.
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Instruction-issue priority of a wave from its progress through its unit:
// 3 until half of the unit's super-tiles are done, 2 until three quarters,
// 1 until seven eighths, then 0.  Two workgroups share a CU and hold equal
// work, but at equal priority issue favours the older waves: the first one
// runs ahead and the second finishes alone with the CU half used.  Dropping
// the leader's priority at these marks lets the other catch up at each one.
__device__ __forceinline__ void progress_prio(int done, int total, int& cur) {
  const int p = 8 * done >= 7 * total ? 0 : (4 * done >= 3 * total ? 1 : (2 * done >= total ? 2 : 3));
  if (p == cur) return;
  cur = p;
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// Workgroup barrier that first drains this wave's LDS reads, so a ring entry
// released at the barrier has no read of it still in flight.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Walsh-Hadamard transform (unnormalized, natural order) of 128 values held
// as 32 per lane, lane quarter q holding values 32q .. 32q + 31: strides 1..16
// inside the lane, 32 and 64 across lane quarters (lanes l ^ 16, l ^ 32).
__device__ __forceinline__ void wht128_quarters(float v[32]) {
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((j & hs) == 0) {
        const float x0 = v[j], x1 = v[j + hs];
        v[j] = x0 + x1;
        v[j + hs] = x0 - x1;
      }
    }
  }
  // strides 32 and 64 (lane quarters q4 ^ 1, q4 ^ 2) through the row swaps:
  // permlane16_swap(v, v) returns (own, partner) in lanes with bit 4 clear
  // and (partner, own) where it is set, permlane32_swap the same for bit 5;
  // so r0 + s * r1, s = -1 where the bit is set, is v + partner in the lower
  // lane of each pair and partner - v in the upper one (exact: one rounding)
  const float s16 = (threadIdx.x & 16) ? -1.f : 1.f, s32 = (threadIdx.x & 32) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
    v[j] = fmaf(s16, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j]), false, false);
    v[j] = fmaf(s32, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
}

// Query operand of one lane (query head h0 + hl of KV head hk, dims of lane
// quarter q4 in each 128-dim head half h, bq[4h .. 4h + 3]): MSE keys rotate
// the query like the keys (sign flip, then the Walsh-Hadamard butterflies:
// strides 1..16 inside the lane, 32 and 64 across lane quarters, and at
// head_dim 256 the stride 128 between the lane's two halves), everything
// scaled by softmax scale * log2(e); the values land in fp16 in the order
// key_operand produces dims.
// Power-of-two scale fi = 2^e of a query head's fp16 operand, from the
// lane's largest |value| (before the scale): the head's maximum over its
// four lane quarters lands in [2^13, 2^14); 1 for an all-zero (or non-finite)
// head.
__device__ __forceinline__ float operand_scale(float lane_absmax) {
  const float mx = quarter_max(lane_absmax);
  if (!(mx > 0.f) || mx == INFINITY) return 1.f;
  const int ex = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);  // biased exponent (0: subnormal)
  const int e = 13 - (max(ex, 1) - 127);                                  // 2^13 <= mx * 2^e < 2^14 (normal mx)
  return __uint_as_float(static_cast<uint32_t>(min(max(e, -126), 126) + 127) << 23);
}

// The lane's raw query words (and, for MSE keys, the rotation signs of its
// dims), loaded apart from the arithmetic so that a workgroup can wait for
// them before it issues its first tile loads and then compute the operand
// while those are in flight: the wait a compiler places before a register's
// first use drains every older vector-memory access, tile loads included.
template <int P>
struct QueryRaw {
  static constexpr int kN = 4 * Preset<P>::kNh;
  u32x4a4 w[kN];                                // FP8: [half][dims 64 h + 16 q4 (+8)]; MSE: [half][8 k]
  f32x4 s[Preset<P>::kFp8 ? 1 : 2 * kN];       // MSE: signs of the dims of w[i], two per word group
};

template <int P>
__device__ __forceinline__ void query_load(const DecodeArgs& a, int b, int hk, int h0, bool live, int hl, int q4,
                                           QueryRaw<P>& r) {
  using T = Preset<P>;
  const uint16_t* qrow =
      a.query + (static_cast<int64_t>(b) * a.num_q_heads + hk * a.group + h0 + (live ? hl : 0)) * T::kDim;
#pragma unroll
  for (int hh = 0; hh < T::kNh; ++hh) {
    if constexpr (T::kFp8 != 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        r.w[4 * hh + 2 * h] = *reinterpret_cast<const u32x4a4*>(qrow + 128 * hh + 64 * h + 16 * q4);
        r.w[4 * hh + 2 * h + 1] = *reinterpret_cast<const u32x4a4*>(qrow + 128 * hh + 64 * h + 16 * q4 + 8);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = 128 * hh + 32 * q4 + 8 * k;
        r.w[4 * hh + k] = *reinterpret_cast<const u32x4a4*>(qrow + d0);
      }
    }
  }
}

// MSE keys: the rotation signs of the lane's dims (the same for every unit,
// so they are loaded before the unit search)
template <int P>
__device__ __forceinline__ void query_signs(const DecodeArgs& a, int q4, QueryRaw<P>& r) {
  if constexpr (Preset<P>::kFp8 == 0) {
#pragma unroll
    for (int hh = 0; hh < Preset<P>::kNh; ++hh)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = 128 * hh + 32 * q4 + 8 * k;
        r.s[2 * (4 * hh + k)] = *reinterpret_cast<const f32x4*>(a.signs + d0);
        r.s[2 * (4 * hh + k) + 1] = *reinterpret_cast<const f32x4*>(a.signs + d0 + 4);
      }
  }
}

// Make the loaded words resident (the compiler waits for them here).
template <int P>
__device__ __forceinline__ void query_wait(const QueryRaw<P>& r) {
#pragma unroll
  for (int i = 0; i < QueryRaw<P>::kN; ++i) asm volatile("" ::"v"(r.w[i].x), "v"(r.w[i].y), "v"(r.w[i].z), "v"(r.w[i].w));
  if constexpr (Preset<P>::kFp8 == 0) {
#pragma unroll
    for (int i = 0; i < 2 * QueryRaw<P>::kN; ++i)
      asm volatile("" ::"v"(r.s[i].x), "v"(r.s[i].y), "v"(r.s[i].z), "v"(r.s[i].w));
  }
}

template <int P>
__device__ __forceinline__ void query_operand(const DecodeArgs& a, const QueryRaw<P>& r, bool live, half8* bq,
                                              float& fi) {
  using T = Preset<P>;
  const bool bf = a.q_bf16 != 0;
  float v[T::kNh][32];
  if constexpr (T::kFp8 != 0) {
    // dims 16*q4 + j (v[j]) and 64 + 16*q4 + j (v[16 + j]) of each half;
    // bq[4h + c][e] = v[h][8c + e]
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4a4 w0 = r.w[4 * hh + 2 * h], w1 = r.w[4 * hh + 2 * h + 1];
      const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[hh][16 * h + 2 * j] = widen16(w[j] & 0xFFFFu, bf);
        v[hh][16 * h + 2 * j + 1] = widen16(w[j] >> 16, bf);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh)
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[hh][j]));
    fi = operand_scale(live ? amax * a.qscale : 0.f);
    const float qs = live ? a.qscale * fi : 0.f;
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(v[hh][8 * c + e] * qs);
      bq[4 * hh + c] = h;
    }
  } else {
    // dims 128*hh + 32*q4 + j (v[hh][j])
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4a4 w = r.w[4 * hh + k];
        const f32x4 s0 = r.s[2 * (4 * hh + k)], s1 = r.s[2 * (4 * hh + k) + 1];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[hh][8 * k + 2 * j] = widen16(ww[j] & 0xFFFFu, bf) * (j < 2 ? s0[2 * j] : s1[2 * j - 4]);
          v[hh][8 * k + 2 * j + 1] = widen16(ww[j] >> 16, bf) * (j < 2 ? s0[2 * j + 1] : s1[2 * j - 3]);
        }
      }
      wht128_quarters(v[hh]);
    }
    if constexpr (T::kNh == 2) {  // stride 128: (lower + upper, lower - upper)
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float x0 = v[0][j], x1 = v[1][j];
        v[0][j] = x0 + x1;
        v[1][j] = x0 - x1;
      }
    }
    // 1/sqrt(head_dim) of the rotation
    const float qs0 = a.qscale * (T::kNh == 2 ? 0.0625f : 0.08838834764831845f);
    float amax = 0.f;
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh)
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[hh][j]));
    fi = operand_scale(live ? amax * qs0 : 0.f);
    const float qs = live ? qs0 * fi : 0.f;
#pragma unroll
    for (int hh = 0; hh < T::kNh; ++hh)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // the dim key_operand holds at (chunk c, element e) of the lane's 32
        const int dd =
            T::kKb == 4 ? tq::key4_dim(c, e) : (T::kKb == 2 ? tq::key2_dim(c, e) : tq::key3_pair_dim(c, e));
        h[e] = static_cast<_Float16>(v[hh][dd] * qs);
      }
      bq[4 * hh + c] = h;
    }
  }
}

// ---- length-balanced units ----

using tq::wave_incl_scan_i;
using tq::wave_max_i;
using tq::wave_sum_i;

struct UnitRange {
  int b;                 // sequence of the unit, -1 if the unit is idle
  int t_begin, t_end;    // its tiles [t_begin, t_end) of sequence b
  int first_u, count_u;  // units of sequence u (the table entry unit u writes; 0, 0 if u >= batch)
  int len;               // seq_lens[b] (0 if the unit is idle)
};

// Every sequence b with tiles_b = ceil(L_b / 16) > 0 gets S_b = ceil(tiles_b
// / tau) units, tau the smallest tile budget with sum_b S_b <= U; its units
// are consecutive and split its tiles evenly (ceil(tiles_b / S_b) each).
// Deterministic, so every workgroup derives the same assignment from
// seq_lens alone; uniform lengths give each sequence U / batch equal units.
// First token a sequence's query attends to: the last `window` tokens
// (itself included), or all of them with no window.
__device__ __forceinline__ int window_start(int seq_len, int window) {
  return window > 0 ? max(0, seq_len - window) : 0;
}

// l0: seq_lens[lane] (0 for lane >= B), loaded by the caller ahead of time.
// Up to 64 sequences each lane keeps its own length in a register; longer
// batches walk seq_lens 64 at a time.  tau is searched between ceil(T / U)
// and the smallest budget known to fit: sum_b ceil(t_b / tau) < T / tau + B,
// so tau = ceil(T / (U - B)) fits whenever U > B (and tau = max_b t_b
// always: one unit per sequence, U >= B).
__device__ __forceinline__ UnitRange find_unit(const int32_t* __restrict__ seq_lens, int l0, int B, int U, int u,
                                               int window) {
  const int lane = threadIdx.x & 63;
  const bool one = B <= 64;  // every length in l0
  auto len_of = [&](int bb) { return bb < B ? seq_lens[bb] : 0; };
  // tiles of a sequence of length L inside its window (tile indices from the window's first tile)
  auto tiles_of = [&](int L) { return L > 0 ? ((L + 15) >> 4) - (window_start(L, window) >> 4) : 0; };
  const int tl0 = tiles_of(l0);
  int T = tl0, tmx = tl0;
  if (!one) {
    for (int bb = lane + 64; bb < B; bb += 64) {
      const int t = tiles_of(len_of(bb));
      T += t;
      tmx = max(tmx, t);
    }
  }
  T = wave_sum_i(T);
  tmx = wave_max_i(tmx);
  int tau = 1;
  if (T > 0) {
    auto units_for = [&](int tt) {
      int c = (tl0 + tt - 1) / tt;
      if (!one)
        for (int bb = lane + 64; bb < B; bb += 64) c += (tiles_of(len_of(bb)) + tt - 1) / tt;
      return wave_sum_i(c);
    };
    int lo = max(1, (T + U - 1) / U), hi = max(lo, tmx);
    if (U > B) hi = max(lo, min(hi, (T + (U - B) - 1) / (U - B)));
    if (units_for(lo) > U) {
      ++lo;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (units_for(mid) <= U)
          hi = mid;
        else
          lo = mid + 1;
      }
    }
    tau = lo;
  }
  UnitRange r{-1, 0, 0, 0, 0, 0};
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int len = b0 == 0 ? l0 : len_of(b0 + lane);
    const int t = b0 == 0 ? tl0 : tiles_of(len);
    const int sb = (t + tau - 1) / tau;
    const int incl = wave_incl_scan_i(sb);
    // (lane indices below are uniform: v_readlane, no LDS crossbar)
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (u >= b0 && u < b0 + 64) {  // table entry of sequence u
      r.first_u = base + __builtin_amdgcn_readlane(incl - sb, u - b0);
      r.count_u = __builtin_amdgcn_readlane(sb, u - b0);
    }
    if (r.b < 0 && u < base + total) {
      const uint64_t m = __ballot(base + incl > u);
      const int lb = __builtin_ctzll(m);  // lane of the unit's sequence
      const int first = base + __builtin_amdgcn_readlane(incl - sb, lb);
      const int nsb = __builtin_amdgcn_readlane(sb, lb);
      const int tb = __builtin_amdgcn_readlane(t, lb);
      const int chunk = (tb + nsb - 1) / nsb;
      r.b = b0 + lb;
      r.len = __builtin_amdgcn_readlane(len, lb);
      r.t_begin = min((u - first) * chunk, tb);
      r.t_end = min(r.t_begin + chunk, tb);
    }
    base += total;
  }
  return r;
}

// Stage 1.  A workgroup owns (unit u: a tile range of one sequence, group of
// G KV heads, up to 16 query heads per KV head) and runs W = G * P waves:
// wave w serves KV head w % G of the group in tile phase w / G.  The range's tiles are staged
// into an LDS ring one super-tile (P consecutive tiles) at a time by the
// whole workgroup, R-1 super-tiles ahead; the phase-p wave of a head scores
// and accumulates tile p of every super-tile from LDS.  At the end the P
// phase waves of a head merge their partial softmax states through LDS and
// the phase-0 wave writes the split's partial rows.  head_dim 256 (two
// halves: twice the accumulators and query operands) runs one tile per wave
// and keeps 2 waves per SIMD's registers.
// Pad (bytes) after each 16-token tile-image row of a contiguous image of
// cache rows of `row` bytes: 16 when the row's dword count is a multiple of
// 8 modulo 64 (the LDS has 64 banks of 4 bytes; 16 rows would fall on 8
// bank groups, rows r and r + 8 colliding), else none.
constexpr uint32_t fix_row_pad(int row) { return ((row / 4) % 64) % 8 == 0 ? 16u : 0u; }

// GATE: the body honours the sparse-V gate vgate (> 0, on exp(s - exact
// running max)); the default kernel is built without its code and keeps a
// single argument, the gated one takes the gate as a second.
//
// FIX: the launch geometry of 8 KV heads at head_dim 128 in combined slots
// (G = Hk = 8, one phase, a two-entry ring of contiguous 16-row tile
// images), fixed at compile time: tile-image offsets fold into the LDS read
// instructions, and the main loop, unrolled over the two ring entries, needs
// no entry arithmetic and no variable wait counts.
template <int P, int TPW, int PACK, int SOA, int GATE, int FIX = 0>
__device__ __forceinline__ void stage1_body(DecodeArgs a, const float vgate) {
  using T = Preset<P>;
  static_assert(T::kNh == 1 || (TPW == 1 && PACK == 0), "head_dim 256: one tile per wave");
  static_assert(!FIX || (T::kNh == 1 && SOA == 0), "fixed geometry: head_dim 128, combined slots");
  constexpr int kOut = 32 * T::kNh;  // output dims per lane (32 of each half)
  extern __shared__ __attribute__((aligned(1024))) uint8_t tq_lds[];
  // dynamic LDS: [3-bit key pair table (3-bit MSE keys only)] [ring]
  constexpr uint32_t kLut = (!T::kFp8 && T::kKb == 3) ? static_cast<uint32_t>(tq::kKey3LutBytes) : 0u;
  uint8_t* const tq_ring = tq_lds + kLut;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = FIX ? 8 : a.G, NP = FIX ? 1 : a.P;
  const int Q = NP * TPW;  // tiles per super-tile
  const int hh = w % G, ph = w / G;
  const int Hk = FIX ? 8 : a.num_kv_heads, Hq = a.num_q_heads, g = a.group;
  int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int hgp = lg % (Hk / G);
  lg /= Hk / G;
  const int hg = lg % a.head_groups;
  const int u = lg / a.head_groups;  // unit
  const int hk = hgp * G + hh;
  const int hl = lane & 15, q4 = lane >> 4;

  // The lengths go out first (the unit search waits on them), then what no
  // unit changes: the rotation signs of the lane's dims and the codebook
  // values (scalar loads, so that no wait on vector memory covers them); the
  // tables built from these wait until the first tiles are in flight.
  const int l0 = lane < a.batch ? a.seq_lens[lane] : 0;
  QueryRaw<P> qraw;
  query_signs<P>(a, q4, qraw);
  const cfloat* cen = (const cfloat*)(a.centroids);
  constexpr int kNk = T::kFp8 ? 0 : (1 << T::kKb), kNv = T::kVlm ? (1 << T::kVb) : 0;
  float ck[kNk > 0 ? kNk : 1], cv[kNv > 0 ? kNv : 1];
#pragma unroll
  for (int i = 0; i < kNk; ++i) ck[i] = cen[i];
#pragma unroll
  for (int i = 0; i < kNv; ++i) cv[i] = cen[kNk + i];

  // ---- unit -> (sequence, tile range): length-balanced split ----
  UnitRange ur = find_unit(a.seq_lens, l0, a.batch, a.num_units, u, a.window);
  // uniform by construction (cross-lane results): tell the compiler
  ur.b = __builtin_amdgcn_readfirstlane(ur.b);
  ur.t_begin = __builtin_amdgcn_readfirstlane(ur.t_begin);
  ur.t_end = __builtin_amdgcn_readfirstlane(ur.t_end);
  ur.first_u = __builtin_amdgcn_readfirstlane(ur.first_u);
  ur.count_u = __builtin_amdgcn_readfirstlane(ur.count_u);
  ur.len = __builtin_amdgcn_readfirstlane(ur.len);
  if (u < a.batch && hgp == 0 && hg == 0 && w == 0 && lane == 0) {  // table entry of sequence u
    a.table[2 * u] = ur.first_u;
    a.table[2 * u + 1] = ur.count_u;
  }
  if (ur.b < 0) return;  // idle unit (uniform over the workgroup)
  const int b = ur.b;
  const int seqlen = ur.len;
  const int wstart = window_start(seqlen, a.window);  // tokens before it are masked out of their tile
  const int t_begin = ur.t_begin + (wstart >> 4);     // absolute tile indices of the sequence
  const int t_end = ur.t_end + (wstart >> 4);
  const int h0 = hg * 16;
  const int geff = min(16, g - h0);
  const int64_t prow0 = static_cast<int64_t>(u) * Hq + hk * g + h0;  // partial row of query head h0
  auto prow = [&](int j) { return prow0 + j; };

  if (t_begin >= t_end) {  // empty range: zero partial, lse = -inf
    if (ph == 0) {
      constexpr int kDimLog2 = T::kNh == 2 ? 8 : 7;
      for (int idx = lane; idx < geff * T::kDim; idx += 64)
        a.part[prow(idx >> kDimLog2) * T::kRow + (idx & (T::kDim - 1))] = 0.f;
      if (lane < geff) a.part[prow(lane) * T::kRow + T::kDim] = -INFINITY;
    }
    return;
  }
  // the query words: issued now, resident before the first tile loads go out
  query_load<P>(a, b, hk, h0, hl < geff, hl, q4, qraw);

  // ---- tile image geometry ----
  ImageGeom geo;
  geo.row = static_cast<uint32_t>(Hk * T::kSlot);
  geo.base = static_cast<uint32_t>(hgp * G * T::kSlot);
  geo.contiguous = FIX ? true : a.contiguous != 0;
  const uint32_t piece = static_cast<uint32_t>(G * T::kSlot);
  // chunks covering row piece r: from its start aligned down to 16 bytes up
  // to its end aligned up, so no chunk crosses the end of its cache block
  auto piece_chunks = [&](int r) { return (((geo.base + r * geo.row) & 15u) + piece + 15u) >> 4; };
  // Fixed geometry: the image rows sit kRowPad bytes apart beyond the cache
  // row, where a cache row's dword count is a multiple of 8 mod 64 (then
  // lanes reading one column of rows r and r + 8 would share LDS banks)
  constexpr uint32_t kRowPad = FIX ? fix_row_pad(8 * T::kSlot) : 0u;
  const uint32_t lrow = geo.row + kRowPad;  // LDS bytes per image row (contiguous images)
  uint32_t tc;  // 16-byte chunks of one tile image
  if (geo.contiguous) {
    tc = lrow;  // 16 rows of `lrow` bytes
  } else {
    tc = 0;
    for (int r = 0; r < 16; ++r) tc += piece_chunks(r);
  }
  // LDS start of token row r: chunk prefix of the rows before it plus the
  // row piece's misalignment
  auto row_start = [&](int r) -> uint32_t {
    if (geo.contiguous) return r * lrow;
    uint32_t c = 0;
    for (int i = 0; i < r; ++i) c += piece_chunks(i);
    return 16 * c + ((geo.base + r * geo.row) & 15u);
  };

  // ---- ring: this wave's DMA slots of each super-tile ----
  constexpr int kSpt8 = (8 * T::kSlot + kRowPad + 63) / 64;  // 1 KB slots of a fixed-geometry tile image
  static_assert(!FIX || kSpt8 == (8 * T::kSlot + 63) / 64, "row pad fits the plan's slots");
  const int spt = FIX ? kSpt8 : a.spt;
  Ring<P, SOA> ring;
  ring.lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tq_ring)));
  ring.entry = static_cast<uint32_t>(Q * spt) * 1024u;
  ring.my_loads = (spt - hh + G - 1) / G;  // per tile
  ring.meta_loads = 0u;
#pragma unroll
  for (int k = 0; k < Ring<P, SOA>::kLoads; ++k) {
    const int n = hh + k * G;  // slot of tile ph (n < spt for k < my_loads)
    ring.dst[k] = static_cast<uint32_t>(ph * TPW * spt + n) * 1024u;  // in tile 0 of this wave's TPW
    if constexpr (SOA != 0) {
      // SoA image: the tile's 16 token rows of data (G rows of kDb bytes
      // each, from one run when G == Hk, else from 16 pieces at the cache's
      // row stride) in the first dslots slots, each image row followed by
      // soa_pad bytes; then its metadata records (16 x G x kMb bytes).  The
      // pad moves the image row stride off multiples of 256 bytes (G * kDb
      // here), where the 16 lanes reading one column of 16 rows would all
      // hit one LDS bank.  A pad chunk repeats the row's last chunk (an L2
      // hit).
      using S = Soa<P>;
      const int ds = a.dslots;
      if (n < ds) {
        const uint32_t pc = static_cast<uint32_t>(G * S::kDb) / 16u;  // chunks of a token row
        const uint32_t pr = pc + static_cast<uint32_t>(a.soa_pad) / 16u;  // chunks of an image row
        const uint32_t p = min(static_cast<uint32_t>(64 * n + lane), 16u * pr - 1u);
        const uint32_t r = p / pr, j = min(p % pr, pc - 1u);
        ring.off[k] = geo.contiguous ? 16u * (r * pc + j)
                                     : r * static_cast<uint32_t>(Hk * S::kDb) +
                                           static_cast<uint32_t>(hgp * G * S::kDb) + 16u * j;
      } else {
        ring.meta_loads |= 1u << k;
        const uint32_t meta_off = static_cast<uint32_t>(a.block_size * Hk * S::kDb);  // region start in a block
        const uint32_t pc = static_cast<uint32_t>(G * S::kMb) / 16u;
        const uint32_t tot = static_cast<uint32_t>(G * S::kMb);  // 16 records of G*kMb bytes = G*kMb chunks
        const uint32_t c = min(static_cast<uint32_t>(64 * (n - ds) + lane), tot - 1u);
        ring.off[k] = meta_off + (geo.contiguous ? 16u * c
                                                 : (c / pc) * static_cast<uint32_t>(Hk * S::kMb) +
                                                       static_cast<uint32_t>(hgp * G * S::kMb) + 16u * (c % pc));
      }
      continue;
    }
    uint32_t c = min(static_cast<uint32_t>(64 * n + lane), tc - 1);
    if (geo.contiguous) {
      if constexpr (kRowPad != 0) {
        // image chunk c = row r, chunk j of lrow / 16; the pad chunks re-read
        // the row's last chunk (an L2 hit)
        const uint32_t rc = lrow / 16u, r = c / rc, j = min(c % rc, geo.row / 16u - 1u);
        ring.off[k] = r * geo.row + 16u * j;
      } else {
        ring.off[k] = 16 * c;
      }
    } else {
      int r = 0;
      uint32_t first = 0;  // first chunk of row r
      for (int i = 0; i < 15; ++i) {
        const uint32_t nc = piece_chunks(r);
        if (c >= first + nc) {
          first += nc;
          ++r;
        }
      }
      ring.off[k] = ((geo.base + r * geo.row) & ~15u) + 16 * (c - first);
    }
  }
  const int R = FIX ? 2 : a.ring_depth;
  const int bs_log2 = 31 - __clz(a.block_size);
  const int64_t blk_bytes = static_cast<int64_t>(a.block_size) * geo.row;
  // Block ids are read with scalar loads (the table is constant while the
  // kernel runs): a vector load here would make the compiler drain every
  // outstanding ring load before its result could be used.
  const cint32* btab = (const cint32*)(a.block_table) + static_cast<int64_t>(b) * a.bt_stride;
  const uint32_t blk_bytes32 = static_cast<uint32_t>(blk_bytes);
  // block id of this wave's tile of super-tile u; tiles past the split's end
  // stand in for its last tile (in bounds; loaded, never computed), so every
  // wave issues the same number of loads per super-tile
  auto my_tile = [&](int u, int j) { return min(t_begin + u * Q + ph * TPW + j, t_end - 1); };
  auto block_of = [&](int t) { return btab[(t * 16) >> bs_log2]; };
  struct Blk {
    int id[TPW];
  };
  auto blocks_of = [&](int u) {
    Blk r;
#pragma unroll
    for (int j = 0; j < TPW; ++j) r.id[j] = block_of(my_tile(u, j));
    return r;
  };
  auto issue = [&](int u, int entry, const Blk& blk) {
    const uint32_t e0 = ring.lds_base + static_cast<uint32_t>(entry) * ring.entry;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = my_tile(u, j);
      const uint8_t* blkp = a.cache + static_cast<uint64_t>(static_cast<uint32_t>(blk.id[j])) * blk_bytes32;
      const uint32_t t16 = static_cast<uint32_t>((t * 16) & (a.block_size - 1));  // tile's first row in the block
      if constexpr (SOA != 0) {
        const uint8_t* bd = blkp + t16 * static_cast<uint32_t>(Hk * Soa<P>::kDb);
        const uint8_t* bm = blkp + t16 * static_cast<uint32_t>(Hk * Soa<P>::kMb);
#pragma unroll
        for (int k = 0; k < Ring<P, SOA>::kLoads; ++k)
          if (k < ring.my_loads)
            dma16(((ring.meta_loads >> k) & 1u) ? bm : bd, ring.off[k],
                  e0 + ring.dst[k] + static_cast<uint32_t>(j * spt) * 1024u);
      } else {
        const uint8_t* base = blkp + t16 * geo.row;
#pragma unroll
        for (int k = 0; k < Ring<P, SOA>::kLoads; ++k)
          if (k < ring.my_loads)
            dma16(base, ring.off[k], e0 + ring.dst[k] + static_cast<uint32_t>(j * spt) * 1024u);
      }
    }
  };
  const int nst = (t_end - t_begin + Q - 1) / Q;
  const int pre = min(R - 1, nst);
  const Blk blk0 = blocks_of(0);
  query_wait<P>(qraw);
  issue(0, 0, blk0);
  for (int d = 1; d < pre; ++d) issue(d, d, blocks_of(d));
  Blk blk_next = blocks_of(R - 1);  // next refill's block ids, fetched a step ahead

  // ---- query operand (registers), computed while the first tiles load ----
  half8 bq[4 * T::kNh];
  float qfi;
  query_operand<P>(a, qraw, hl < geff, bq, qfi);
  if constexpr (PACK != 0) {  // columns 8..15 carry tile B's scores of head c - 8: its units
    const float fb = swap8(qfi);
    if (hl >= 8) qfi = fb;
  }

  // fp16 codebooks for the byte-permute lookups: keys (la, lb), Lloyd-Max
  // values (lv, the value codebook after the key codebook in the table)
  auto lut_bytes = [](const uint32_t* hb, int base, int shift) {
    return ((hb[base] >> shift) & 0xFF) | (((hb[base + 1] >> shift) & 0xFF) << 8) |
           (((hb[base + 2] >> shift) & 0xFF) << 16) | (((hb[base + 3] >> shift) & 0xFF) << 24);
  };
  tq::Lut8 la{}, lb{};
  ValLut lv{};
  if constexpr (kNk > 0) {
    uint32_t hb[16] = {};
#pragma unroll
    for (int i = 0; i < kNk; ++i) hb[i] = __half_as_ushort(__float2half_rn(ck[i]));
    la = {lut_bytes(hb, 0, 0), lut_bytes(hb, 4, 0), lut_bytes(hb, 0, 8), lut_bytes(hb, 4, 8)};
    if (T::kKb == 4) lb = {lut_bytes(hb, 8, 0), lut_bytes(hb, 12, 0), lut_bytes(hb, 8, 8), lut_bytes(hb, 12, 8)};
  }
  if constexpr (kNv > 0) {
    uint32_t hv[16] = {};
#pragma unroll
    for (int i = 0; i < kNv; ++i) hv[i] = __half_as_ushort(__float2half_rn(cv[i]));
    lv.lo = {lut_bytes(hv, 0, 0), lut_bytes(hv, 4, 0), lut_bytes(hv, 0, 8), lut_bytes(hv, 4, 8)};
    if (T::kVb == 4) lv.hi = {lut_bytes(hv, 8, 0), lut_bytes(hv, 12, 0), lut_bytes(hv, 8, 8), lut_bytes(hv, 12, 8)};
  }
  // 3-bit keys: the pair table, entry f = (c[f & 7], c[f >> 3]) in fp16 at
  // dword 64 f + copy (one copy per lane), written four equal copies at a
  // time; the main loop's first barrier orders these writes before any lookup
  if constexpr (kLut != 0) {
    f32x4* lut = reinterpret_cast<f32x4*>(tq_lds);
    constexpr int kPer = tq::kKey3LutCopies / 4;  // 16-byte writes per entry
    for (int i = static_cast<int>(threadIdx.x); i < 64 * kPer; i += static_cast<int>(blockDim.x)) {
      const uint32_t f = static_cast<uint32_t>(i / kPer);
      uint32_t pair, unused;
      tq::lut8((f & 7u) | ((f >> 3) << 8), la, pair, unused);  // (c[f & 7], c[f >> 3])
      const float x = __uint_as_float(pair);
      lut[i] = f32x4{x, x, x, x};
    }
  }
  // LDS address of this lane's copy of table entry 0: the kernels declare no
  // static LDS (the launcher checks), so the dynamic block starts at 0
  const uint32_t klane = 4u * static_cast<uint32_t>(lane);
  LaneOff<P> off;
  if constexpr (SOA != 0) {
    using S = Soa<P>;
    off.sd = static_cast<uint32_t>(G * S::kDb + a.soa_pad);  // image row: G data rows + the pad
    off.sm = static_cast<uint32_t>(G * S::kMb);
    off.k = hl * off.sd + static_cast<uint32_t>(hh * S::kDb) +
            static_cast<uint32_t>(T::kFp8 ? 16 * q4 : 4 * T::kKb * q4);
    off.ksh = 0u;
    off.mo[0] = static_cast<uint32_t>(4 * q4) * off.sd + static_cast<uint32_t>(hh * S::kDb);
    off.mo[1] = off.mo[2] = off.mo[3] = 0u;
    off.vcol = static_cast<uint32_t>(T::kKdata + T::kVb * hl);
    off.mm0 = static_cast<uint32_t>(a.dslots) * 1024u + static_cast<uint32_t>(4 * q4) * off.sm +
              static_cast<uint32_t>(hh * S::kMb);
  } else {
    const uint32_t kraw = row_start(hl) + static_cast<uint32_t>(hh * T::kSlot) +
                          static_cast<uint32_t>(T::kFp8 ? 16 * q4 : 4 * T::kKb * q4);
    off.k = kraw & ~3u;
    off.ksh = kraw & 3u;
#pragma unroll
    for (int i = 0; i < 4; ++i) off.mo[i] = row_start(4 * q4 + i) + static_cast<uint32_t>(hh * T::kSlot);
    off.vcol = static_cast<uint32_t>(T::kKps + T::kVb * hl);
    off.mm0 = off.sd = off.sm = 0u;
  }

  Softmax sm{-INFINITY, 0.f, 0.f, 1.f / qfi, qfi, -INFINITY, -INFINITY};
  const float vglg = GATE ? __log2f(vgate) : 0.f;  // log2 of the sparse-V gate
  f32x4 acc[8 * T::kNh];
#pragma unroll
  for (int n = 0; n < 8 * T::kNh; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  PendingTile<P> pend;
  bool have_pend = false;

  // ---- main loop: wait for super-tile u, release the entry of u-1, refill
  // it with u+R-1, compute this wave's tile(s) of u from the entry at ent ----
  auto compute = [&](int u, const uint8_t* ent) {
    if constexpr (PACK != 0) {
      // the wave's two tiles of the super-tile, scored together
      const int t = t_begin + u * Q + ph * TPW;
      if (t < t_end) {
        const uint8_t* img = ent + static_cast<uint32_t>(ph * TPW * spt) * 1024u;
        score_pair_packed<P, SOA>(img, img + static_cast<uint32_t>(spt) * 1024u, off, la, lb, lv, klane, bq,
                                  min(16, seqlen - t * 16), t + 1 < t_end ? min(16, seqlen - (t + 1) * 16) : 0,
                                  max(0, wstart - t * 16), max(0, wstart - (t + 1) * 16), vgate, vglg, sm, acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int t = t_begin + u * Q + ph * TPW + j;
        if (t < t_end) {
          TileRegs<P> r;
          const uint8_t* img = ent + static_cast<uint32_t>((ph * TPW + j) * spt) * 1024u;
          load_tile<P, SOA>(img, off, r);
          PendingTile<P> cur;
          score_tile<P, SOA>(r, off, la, lb, klane, bq, min(16, seqlen - t * 16), max(0, wstart - t * 16), vgate,
                             vglg, sm, acc, pend, have_pend, cur);
          if (have_pend) {
            if (!GATE || pair_has_values(pend, cur)) accumulate_pair<P>(pend, cur, lv, acc);
            have_pend = false;
          } else {
            pend = cur;
            have_pend = true;
          }
        }
      }
    }
  };
  if constexpr (FIX != 0) {
    // two entries: super-tile u in entry u & 1; this wave's loads of u + 1 are
    // its only ones in flight once u has arrived
    constexpr uint32_t kEntry = static_cast<uint32_t>(TPW * kSpt8) * 1024u;
    int prio = -1;
    for (int u = 0; u < nst; u += 2) {
      progress_prio(u, nst, prio);
      vm_wait(0);
      wg_barrier();
      if (u + 1 < nst) {
        issue(u + 1, 1, blk_next);
        blk_next = blocks_of(u + 2);
      }
      compute(u, tq_ring);
      if (u + 1 >= nst) break;
      vm_wait(0);
      wg_barrier();
      if (u + 2 < nst) {
        issue(u + 2, 0, blk_next);
        blk_next = blocks_of(u + 3);
      }
      compute(u + 1, tq_ring + kEntry);
    }
  } else {
    int entry = 0;
    int prio = -1;
    for (int u = 0; u < nst; ++u) {
      progress_prio(u, nst, prio);
      vm_wait(TPW * ring.my_loads * min(R - 2, nst - 1 - u));
      wg_barrier();
      if (u + R - 1 < nst) {
        issue(u + R - 1, entry == 0 ? R - 1 : entry - 1, blk_next);
        blk_next = blocks_of(u + R);
      }
      compute(u, tq_ring + static_cast<uint32_t>(entry) * ring.entry);
      entry = entry + 1 == R ? 0 : entry + 1;
    }
  }

  if (have_pend) {  // an odd tile out: pair it with an empty one
    PendingTile<P> none;
#pragma unroll
    for (int h = 0; h < T::kNh; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) none.vw[h][i] = 0u;
    none.pv = half4{0, 0, 0, 0};
    if (!GATE || pair_has_values(pend, none)) accumulate_pair<P>(pend, none, lv, acc);
  }

  // ---- this wave's normalized partial (output / l, base-2 LSE) ----
  if (PACK != 0) {  // lanes c and c ^ 8 summed the two tiles of each pair: add them
    sm.l += swap8(sm.l);
    sm.z += swap8(sm.z);
  }
  const float l_run = quarter_sum(sm.l), z_run = quarter_sum(sm.z);
  float o[kOut];  // o[32 * h + 8 * i + n]: acc[8 * h + n][i] as output
  {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int h = 0; h < T::kNh; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int pos = T::kVb == 4 ? tq::val4_pos(n) : (T::kVb == 3 ? tq::val3_pos(n) : tq::val2_pos(n));
        const float x = acc[8 * h + n][i];
        o[32 * h + 8 * i + n] = T::kVlm ? x * inv : fmaf(x, static_cast<float>(1u << (24 - pos)), z_run) * inv;
      }
    }
  }
  float lse2 = l_run > 0.f ? sm.m + log2f(l_run) : -INFINITY;

  // ---- merge the P phase waves of each head (through LDS) ----
  if (NP > 1) {
    wg_barrier();  // every wave is done with the ring
    float* mrg = reinterpret_cast<float*>(tq_ring);
    if (ph > 0) {
      float* reg = mrg + ((ph - 1) * G + hh) * ((kOut + 1) * 64);
#pragma unroll
      for (int k = 0; k < kOut; ++k) reg[k * 64 + lane] = o[k];
      reg[kOut * 64 + lane] = lse2;
    }
    wg_barrier();
    if (ph == 0) {
      float M = lse2;
      for (int p = 1; p < NP; ++p) M = fmaxf(M, mrg[((p - 1) * G + hh) * ((kOut + 1) * 64) + kOut * 64 + lane]);
      float wsum = __builtin_amdgcn_exp2f(lse2 - M);
#pragma unroll
      for (int k = 0; k < kOut; ++k) o[k] *= wsum;
      for (int p = 1; p < NP; ++p) {
        const float* reg = mrg + ((p - 1) * G + hh) * ((kOut + 1) * 64);
        const float lp = reg[kOut * 64 + lane];
        if (lp == -INFINITY) continue;
        const float wp = __builtin_amdgcn_exp2f(lp - M);
        wsum += wp;
#pragma unroll
        for (int k = 0; k < kOut; ++k) o[k] = fmaf(wp, reg[k * 64 + lane], o[k]);
      }
      const float inv = 1.f / wsum;
#pragma unroll
      for (int k = 0; k < kOut; ++k) o[k] *= inv;
      lse2 = M + log2f(wsum);
    }
  }

  // ---- Lloyd-Max values were accumulated in the rotated space: rotate the
  // head's output back, o <- s .* (H o) / sqrt(D) (lane quarter q4 holds dims
  // 128 h + 32 q4 .. 128 h + 32 q4 + 31 of each half h, as in the query
  // operand; at head_dim 256 the stride-128 butterfly joins the halves) ----
  if constexpr (T::kVlm != 0) {
    if (ph == 0) {
#pragma unroll
      for (int h = 0; h < T::kNh; ++h) wht128_quarters(o + 32 * h);
      if constexpr (T::kNh == 2) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float x0 = o[j], x1 = o[32 + j];
          o[j] = x0 + x1;
          o[32 + j] = x0 - x1;
        }
      }
      constexpr float kInvSqrtD = T::kNh == 2 ? 0.0625f : 0.08838834764831845f;
#pragma unroll
      for (int h = 0; h < T::kNh; ++h) {
        const float* sp = a.signs + 128 * h + 32 * q4;
#pragma unroll
        for (int j = 0; j < 32; ++j) o[32 * h + j] *= sp[j] * kInvSqrtD;
      }
    }
  }

  // ---- the split's partial rows: output and natural-log LSE ----
  if (ph == 0 && hl < geff) {
#pragma unroll
    for (int h = 0; h < T::kNh; ++h) {
      float* orow = a.part + prow(hl) * T::kRow + 128 * h + 32 * q4;
      const float* oh = o + 32 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<f32x4*>(orow + 8 * i) = f32x4{oh[8 * i], oh[8 * i + 1], oh[8 * i + 2], oh[8 * i + 3]};
        *reinterpret_cast<f32x4*>(orow + 8 * i + 4) =
            f32x4{oh[8 * i + 4], oh[8 * i + 5], oh[8 * i + 6], oh[8 * i + 7]};
      }
    }
    if (q4 == 0) a.part[prow(hl) * T::kRow + T::kDim] = lse2 * kLn2;
  }
}

template <int P, int TPW, int PACK, int SOA, int FIX>
__global__ __launch_bounds__(512, Preset<P>::kNh == 2 ? 2 : 4) void tq_decode_stage1_kernel(DecodeArgs a) {
  stage1_body<P, TPW, PACK, SOA, 0, FIX>(a, 0.f);
}

template <int P, int TPW, int PACK, int SOA, int FIX>
__global__ __launch_bounds__(512, Preset<P>::kNh == 2 ? 2 : 4) void tq_decode_stage1_gated_kernel(DecodeArgs a,
                                                                                                   float value_gate) {
  stage1_body<P, TPW, PACK, SOA, 1, FIX>(a, value_gate);
}

// ---------------------------------------------------------------- stage 2

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Output = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max), lse = max
// + log(sum_s w_s), over the units of a (sequence, query head) row (the table
// stage 1 writes).  Latency-bound, so the loads are issued together: after
// the table read each lane fetches its 2 output dims of each 128-dim head
// half (NH halves) of up to 16 units and lane j the LSE of unit j, all at
// once.  kW waves share a row (wave w takes units w, w + kW, ...; their
// running (max, sum, output) combine through LDS) when rows have many
// units; otherwise each wave of the workgroup takes its own row (kW = 1).
template <int kW, int NH>
__global__ __launch_bounds__(kW > 4 ? 64 * kW : 256) void tq_decode_stage2_kernel(const int32_t* __restrict__ table,
                                                               const float* __restrict__ part, int Hq, int rows,
                                                               void* out, int out_dtype, float* lse_out,
                                                               const float* __restrict__ sinks) {
  constexpr int kBatch = 16;
  constexpr int kDim = 128 * NH, kRowN = kDim + static_cast<int>(tq::kPartPad), kO = 2 * NH;
  __shared__ float comb[kW > 1 ? kW - 1 : 1][kO * 64 + 2];
  const int lane = threadIdx.x & 63;
  const int w = kW > 1 ? (threadIdx.x >> 6) : 0;
  const int row = kW > 1 ? blockIdx.x : blockIdx.x * 4 + (threadIdx.x >> 6);
  if (kW == 1 && row >= rows) return;
  const int b = row / Hq, hq = row - b * Hq;
  const int first = table[2 * b], n = table[2 * b + 1];
  const float* base = part + (static_cast<int64_t>(first) * Hq + hq) * kRowN;
  const int64_t stride = static_cast<int64_t>(Hq) * kRowN * kW;  // between this wave's consecutive units
  base += static_cast<int64_t>(w) * Hq * kRowN;
  const int nw = n > w ? (n - w + kW - 1) / kW : 0;  // units of this wave
  float M = -INFINITY, den = 0.f;
  float o[kO];  // dims 128 h + 2 lane, 128 h + 2 lane + 1 at o[2 h], o[2 h + 1]
#pragma unroll
  for (int k = 0; k < kO; ++k) o[k] = 0.f;
  for (int s0 = 0; s0 < nw; s0 += kBatch) {
    const int ns = min(kBatch, nw - s0);
    float2 v[kBatch][NH];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        v[q][h] = q < ns ? *reinterpret_cast<const float2*>(base + (s0 + q) * stride + 128 * h + 2 * lane)
                         : make_float2(0.f, 0.f);
    const float ls = lane < ns ? base[(s0 + lane) * stride + kDim] : -INFINITY;
    float Mb = ls;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) Mb = fmaxf(Mb, __shfl_xor(Mb, m, 64));  // lanes 0..15 hold the batch
    Mb = __shfl(Mb, 0, 64);
    const float Mn = fmaxf(M, Mb);
    if (Mn == -INFINITY) continue;  // nothing live yet
    const float alpha = M == -INFINITY ? 0.f : expf(M - Mn);
#pragma unroll
    for (int k = 0; k < kO; ++k) o[k] *= alpha;
    den *= alpha;
    M = Mn;
    const float wl = ls == -INFINITY ? 0.f : expf(ls - M);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), q));
      den += wq;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        o[2 * h] = fmaf(wq, v[q][h].x, o[2 * h]);
        o[2 * h + 1] = fmaf(wq, v[q][h].y, o[2 * h + 1]);
      }
    }
  }
  if (kW > 1) {
    if (w > 0) {
#pragma unroll
      for (int k = 0; k < kO; ++k) comb[w - 1][kO * lane + k] = o[k];
      if (lane == 0) {
        comb[w - 1][kO * 64] = M;
        comb[w - 1][kO * 64 + 1] = den;
      }
    }
    __syncthreads();
    if (w != 0) return;
  }
  float Mt = M;
#pragma unroll
  for (int k = 0; k < kW - 1; ++k) Mt = fmaxf(Mt, comb[k][kO * 64]);  // no-op for kW == 1
  // an attention sink: one more term of the denominator, with no value
  const float sink = sinks ? sinks[hq] : -INFINITY;
  Mt = fmaxf(Mt, sink);
  float lse = -INFINITY;
  if (Mt != -INFINITY) {
    const float a0 = M == -INFINITY ? 0.f : expf(M - Mt);
#pragma unroll
    for (int k = 0; k < kO; ++k) o[k] *= a0;
    den *= a0;
#pragma unroll
    for (int k = 0; k < kW - 1; ++k) {
      const float mk = comb[k][kO * 64];
      if (mk == -INFINITY) continue;
      const float ak = expf(mk - Mt);
      den = fmaf(ak, comb[k][kO * 64 + 1], den);
#pragma unroll
      for (int j = 0; j < kO; ++j) o[j] = fmaf(ak, comb[k][kO * lane + j], o[j]);
    }
    if (sink != -INFINITY) den += expf(sink - Mt);
#pragma unroll
    for (int k = 0; k < kO; ++k) o[k] /= den;
    lse = Mt + logf(den);
  } else {
#pragma unroll
    for (int k = 0; k < kO; ++k) o[k] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int64_t ob = static_cast<int64_t>(row) * kDim + 128 * h + 2 * lane;
    const float o0 = o[2 * h], o1 = o[2 * h + 1];
    if (out_dtype == TQ_F32) {
      *reinterpret_cast<float2*>(static_cast<float*>(out) + ob) = make_float2(o0, o1);
    } else if (out_dtype == TQ_F16) {
      *reinterpret_cast<__half2*>(static_cast<__half*>(out) + ob) =
          __halves2half2(__float2half_rn(o0), __float2half_rn(o1));
    } else {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + ob) =
          static_cast<uint32_t>(f32_to_bf16_rne(o0)) | (static_cast<uint32_t>(f32_to_bf16_rne(o1)) << 16);
    }
  }
  if (lse_out && lane == 0) lse_out[row] = lse;
}

constexpr int kMaxLds = 160 * 1024;

template <int P, int TPW, int PACK, int SOA, int GATE, int FIX>
int launch_stage1_g(const DecodeArgs& a, float gate, int64_t nblocks, size_t lds, hipStream_t stream) {
  const void* fn = GATE ? reinterpret_cast<const void*>(&tq_decode_stage1_gated_kernel<P, TPW, PACK, SOA, FIX>)
                        : reinterpret_cast<const void*>(&tq_decode_stage1_kernel<P, TPW, PACK, SOA, FIX>);
  const int st = tq::set_max_lds_once(fn, kMaxLds);
  if (st != TQ_OK) return st;
  DecodeArgs arg = a;
  float g = gate;
  void* args[] = {&arg, &g};  // the default kernel reads the first only
  return tq::hip_status(
      hipLaunchKernel(fn, dim3(static_cast<unsigned>(nblocks)), dim3(64 * a.G * a.P), args, lds, stream));
}

// The sparse-V gate takes its own kernels; 8 KV heads at head_dim 128 in
// combined slots with a two-entry ring take the fixed-geometry ones.
template <int P, int TPW, int PACK, int SOA>
int launch_stage1_t(const DecodeArgs& a, float gate, int64_t nblocks, size_t lds, hipStream_t stream) {
  constexpr bool kCanFix = Preset<P>::kNh == 1 && SOA == 0;
  const bool fix = kCanFix && a.G == 8 && a.num_kv_heads == 8 && a.P == 1 && a.ring_depth == 2 &&
                   a.contiguous != 0 && a.spt == (8 * Preset<P>::kSlot + 63) / 64;
  if (fix) {
    if constexpr (kCanFix)
      return gate > 0.f ? launch_stage1_g<P, TPW, PACK, SOA, 1, 1>(a, gate, nblocks, lds, stream)
                        : launch_stage1_g<P, TPW, PACK, SOA, 0, 1>(a, gate, nblocks, lds, stream);
  }
  return gate > 0.f ? launch_stage1_g<P, TPW, PACK, SOA, 1, 0>(a, gate, nblocks, lds, stream)
                    : launch_stage1_g<P, TPW, PACK, SOA, 0, 0>(a, gate, nblocks, lds, stream);
}

// Two tiles per wave: GQA groups of at most 8 query heads score them packed
// into one MFMA block layout; wider groups one at a time.
template <int P, int SOA>
int launch_stage1_l(const DecodeArgs& a, float gate, int tpw, int64_t nblocks, size_t lds, hipStream_t stream) {
  if (tpw == 2)
    return a.group <= 8 ? launch_stage1_t<P, 2, 1, SOA>(a, gate, nblocks, lds, stream)
                        : launch_stage1_t<P, 2, 0, SOA>(a, gate, nblocks, lds, stream);
  return launch_stage1_t<P, 1, 0, SOA>(a, gate, nblocks, lds, stream);
}

// head_dim 256 (preset code P | kHead256): one tile per wave (the plan's
// choice there: two tile images per wave do not fit the ring).
template <int P>
int launch_stage1(const DecodeArgs& a, float gate, int tpw, bool soa, bool d256, int64_t nblocks, size_t lds,
                  hipStream_t stream) {
  if (d256) {
    if (tpw != 1) return TQ_EUNSUPPORTED;
    return soa ? launch_stage1_t<P | kHead256, 1, 0, 1>(a, gate, nblocks, lds, stream)
               : launch_stage1_t<P | kHead256, 1, 0, 0>(a, gate, nblocks, lds, stream);
  }
  return soa ? launch_stage1_l<P, 1>(a, gate, tpw, nblocks, lds, stream)
             : launch_stage1_l<P, 0>(a, gate, tpw, nblocks, lds, stream);
}

int stage1(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
           int32_t num_kv_heads, const void* kv_cache, int32_t block_size, const int32_t* block_table,
           int32_t block_table_stride, const int32_t* seq_lens, const float* signs, const float* centroids,
           float scale, int32_t num_kv_splits, int32_t sliding_window, float value_gate, void* workspace,
           hipStream_t stream) {
  DecodeArgs a;
  a.window = sliding_window;
  a.query = static_cast<const uint16_t*>(query);
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.signs = signs;
  a.centroids = centroids;
  a.table = static_cast<int32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + tq::table_bytes(batch));
  a.qscale = scale * kLog2e;
  a.q_bf16 = q_dtype == TQ_BF16;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_groups = (a.group + 15) / 16;
  a.block_size = block_size;
  a.bt_stride = block_table_stride;
  a.batch = batch;
  tq::DecodePlan plan;
  // tiles of the longest possible sequence (block-table width), or of a window
  int64_t max_tiles = (static_cast<int64_t>(block_table_stride) * block_size + 15) / 16;
  if (sliding_window > 0) max_tiles = std::min<int64_t>(max_tiles, (sliding_window + 15) / 16 + 1);
  const int st = tq::decode_plan(layout, batch, num_q_heads, num_kv_heads, num_kv_splits, max_tiles, &plan);
  if (st != TQ_OK) return st;
  a.num_units = static_cast<int32_t>(plan.units);
  a.G = plan.G;
  a.P = plan.P;
  a.ring_depth = plan.R;
  a.spt = plan.spt;
  a.contiguous = plan.contiguous;
  a.dslots = plan.dslots;
  a.soa_pad = plan.soa_pad;
  const int64_t nblocks = plan.grid;
  const size_t lds = plan.lds;
  const bool soa = layout->block_layout == TQ_LAYOUT_SOA;
  const bool d256 = layout->head_dim == 256;
  switch (layout->preset) {
    case TQ_K8V4: return launch_stage1<TQ_K8V4>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_4BIT_NC: return launch_stage1<TQ_4BIT_NC>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_K3V4_NC: return launch_stage1<TQ_K3V4_NC>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_3BIT_NC: return launch_stage1<TQ_3BIT_NC>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_K8V3: return launch_stage1<TQ_K8V3>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_K4V3_NC: return launch_stage1<TQ_K4V3_NC>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_2BIT_NC: return launch_stage1<TQ_2BIT_NC>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_K8V3LM: return launch_stage1<TQ_K8V3LM>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_3BIT_LM: return launch_stage1<TQ_3BIT_LM>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_K8V4LM: return launch_stage1<TQ_K8V4LM>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_4BIT_LM: return launch_stage1<TQ_4BIT_LM>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
    case TQ_2BIT_LM: return launch_stage1<TQ_2BIT_LM>(a, value_gate, plan.tpw, soa, d256, nblocks, lds, stream);
  }
  return TQ_EPRESET;
}

template <int NH>
int stage2_t(int32_t batch, int32_t num_q_heads, int32_t num_kv_splits, const float* sinks, const void* workspace,
             void* out, int32_t out_dtype, float* lse_out, hipStream_t stream) {
  int rows = batch * num_q_heads;
  int Hq = num_q_heads;
  const int32_t* table = static_cast<const int32_t*>(workspace);
  const float* part = reinterpret_cast<const float*>(static_cast<const uint8_t*>(workspace) + tq::table_bytes(batch));
  void* args[] = {&table, &part, &Hq, &rows, &out, &out_dtype, &lse_out, &sinks};
  // Rows of many units share several waves (each wave loads up to 16 units
  // at once, so a row of S_max units takes one round of loads); otherwise
  // one wave per row, four rows per workgroup.  S_max is the units of a
  // sequence of a uniform batch (balanced units give long sequences of a
  // ragged one more, which take further rounds).
  const int64_t smax = tq::max_splits(batch, num_kv_splits);
  const void* fn;
  int waves;
  if (smax > 64) {
    fn = reinterpret_cast<const void*>(smax > 128 ? &tq_decode_stage2_kernel<16, NH> : &tq_decode_stage2_kernel<8, NH>);
    waves = smax > 128 ? 16 : 8;
  } else if (smax > 16) {
    fn = reinterpret_cast<const void*>(&tq_decode_stage2_kernel<4, NH>);
    waves = 4;
  } else {
    return tq::hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&tq_decode_stage2_kernel<1, NH>),
                                          dim3((rows + 3) / 4), dim3(256), args, 0, stream));
  }
  return tq::hip_status(hipLaunchKernel(fn, dim3(rows), dim3(64 * waves), args, 0, stream));
}

int stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits, const float* sinks,
           const void* workspace, void* out, int32_t out_dtype, float* lse_out, hipStream_t stream) {
  return head_dim == 256
             ? stage2_t<2>(batch, num_q_heads, num_kv_splits, sinks, workspace, out, out_dtype, lse_out, stream)
             : stage2_t<1>(batch, num_q_heads, num_kv_splits, sinks, workspace, out, out_dtype, lse_out, stream);
}

}  // namespace

namespace tq {
namespace {
thread_local hipError_t g_last_hip_error = hipSuccess;
}
int hip_status(int e) {
  if (e == hipSuccess) return TQ_OK;
  g_last_hip_error = static_cast<hipError_t>(e);
  return TQ_EHIP;
}
}  // namespace tq

extern "C" const char* tq_last_hip_error(void) { return hipGetErrorString(tq::g_last_hip_error); }

namespace tq {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_setup_mutex;
std::vector<std::pair<const void*, int>> g_lds_set;  // (kernel, device) pairs already set up
void* g_scratch_addr[kMaxDevices] = {};             // device address of `scratch`, per device
}  // namespace

int set_max_lds_once(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  std::lock_guard<std::mutex> lock(g_setup_mutex);
  for (const auto& kv : g_lds_set)
    if (kv.first == fn && kv.second == dev) return TQ_OK;
  // the 3-bit key table sits at LDS address 0: no static LDS before the
  // dynamic block
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return hip_status(e);
  if (attr.sharedSizeBytes != 0) return TQ_EUNSUPPORTED;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return hip_status(e);
  g_lds_set.emplace_back(fn, dev);
  return TQ_OK;
}
}  // namespace tq

// Scratch of tq_decode_attention_noalloc: the stage-1 sequence table and
// partial rows that tq_decode_attention keeps in its caller's workspace.  In
// host code `scratch` is only a stand-in for the symbol; kernels get the
// device address looked up below.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of `scratch` on the current device, looked up on the first
// call with that device current and cached per device.
int scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tq::hip_status(e);
  if (dev < 0 || dev >= tq::kMaxDevices) return TQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(tq::g_setup_mutex);
  if (!tq::g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return tq::hip_status(e);
    if (!p) return TQ_EHIP;
    tq::g_scratch_addr[dev] = p;
  }
  *addr = tq::g_scratch_addr[dev];
  return TQ_OK;
}
}  // namespace

extern "C" int tq_decode_stage1(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks,
                                int32_t block_size, const int32_t* block_table, int32_t block_table_stride,
                                const int32_t* seq_lens, const float* signs, const float* centroids, float scale,
                                int32_t num_kv_splits, int32_t sliding_window, float value_gate, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int st = tq::validate_decode(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                               block_size, block_table, block_table_stride, seq_lens, signs, centroids,
                               num_kv_splits, sliding_window, value_gate, workspace, workspace_bytes);
  if (st != TQ_OK || batch == 0) return st;
  return stage1(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, block_size, block_table,
                block_table_stride, seq_lens, signs, centroids, scale, num_kv_splits, sliding_window, value_gate,
                workspace, static_cast<hipStream_t>(stream));
}

extern "C" int tq_decode_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                                const float* sinks, const void* workspace, size_t workspace_bytes, void* out,
                                int32_t out_dtype, float* lse_out, void* stream) {
  int st = tq::validate_stage2(batch, num_q_heads, head_dim, num_kv_splits, workspace, workspace_bytes, out,
                               out_dtype);
  if (st != TQ_OK || batch == 0) return st;
  return stage2(batch, num_q_heads, head_dim, num_kv_splits, sinks, workspace, out, out_dtype, lse_out,
                static_cast<hipStream_t>(stream));
}

extern "C" int tq_decode_attention(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache,
                                   int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                                   int32_t block_table_stride, const int32_t* seq_lens, const float* signs,
                                   const float* centroids, float scale, int32_t num_kv_splits,
                                   int32_t sliding_window, float value_gate, const float* sinks, void* workspace,
                                   size_t workspace_bytes, void* out, int32_t out_dtype, float* lse_out,
                                   void* stream) {
  int st = tq_decode_validate(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                              block_size, block_table, block_table_stride, seq_lens, signs, centroids, num_kv_splits,
                              sliding_window, value_gate, workspace, workspace_bytes, out, out_dtype);
  if (st != TQ_OK || batch == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = stage1(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, block_size, block_table,
              block_table_stride, seq_lens, signs, centroids, scale, num_kv_splits, sliding_window, value_gate,
              workspace, s);
  if (st != TQ_OK) return st;
  return stage2(batch, num_q_heads, layout->head_dim, num_kv_splits, sinks, workspace, out, out_dtype, lse_out, s);
}

extern "C" int tq_decode_attention_noalloc(const tq_layout* layout, const void* query, int32_t q_dtype,
                                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                           const void* kv_cache, int64_t num_blocks, int32_t block_size,
                                           const int32_t* block_table, int32_t block_table_stride,
                                           const int32_t* seq_lens, const float* signs, const float* centroids,
                                           float scale, int32_t num_kv_splits, int32_t sliding_window,
                                           float value_gate, const float* sinks, void* out, int32_t out_dtype,
                                           float* lse_out, void* stream) {
  // Every argument is checked against the scratch capacity before the
  // scratch is looked up (a 256-aligned stand-in address takes the place of
  // the workspace in the host-only check; it is never dereferenced).
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  int st = tq_decode_validate(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                              block_size, block_table, block_table_stride, seq_lens, signs, centroids, num_kv_splits,
                              sliding_window, value_gate, stand_in, TQ_NOALLOC_SCRATCH_BYTES, out, out_dtype);
  if (st != TQ_OK || batch == 0) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = stage1(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, block_size, block_table,
              block_table_stride, seq_lens, signs, centroids, scale, num_kv_splits, sliding_window, value_gate, ws, s);
  if (st != TQ_OK) return st;
  return stage2(batch, num_q_heads, layout->head_dim, num_kv_splits, sinks, ws, out, out_dtype, lse_out, s);
}
