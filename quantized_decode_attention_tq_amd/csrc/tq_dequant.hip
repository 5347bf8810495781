// tq_dequant_kv: the cached prefix of one sequence back to dense K/V in the
// original space, the first step of a continuation prefill ([API]
// _continuation_prefill: dequantize the cached K/V, inverse-rotate MSE keys,
// then attend over cached + new tokens).
//
// Work mapping as in the store (gfx950, wave64): a "row" is one (token, KV
// head) slot, D / 16 lanes per row (8 at head_dim 128, 16 at 256), 16
// consecutive coordinates per lane.  MSE keys: the lane looks up gamma * c[code] for its 16 rotated
// coordinates and applies the rotation's transpose in registers, s .* (H y)
// / sqrt(D) (H symmetric, H H = D I), with the store's butterflies.  FP8 keys
// and the values decode lane-locally.  Each lane writes its 16 outputs of K
// and of V as 16-byte vector stores, so a row's lanes write one contiguous
// run.  HBM-bound: slot bytes in, 2 * D elements out per slot.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "tq.h"
#include "tq_internal.h"
#include "tq_wht.h"

namespace {

constexpr int kDpl = tq::kWhtPerLane;  // coordinates per lane
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct DequantArgs {
  const uint8_t* cache;
  const int32_t* block_table;
  const float* signs;
  const float* centroids;
  void* key_out;
  void* value_out;
  int64_t out_tok_stride;  // elements between consecutive tokens of the outputs
  int32_t num_rows;        // num_tokens * num_kv_heads (< 2^31)
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t slot_bytes;  // slot_size_aligned
  int32_t soa;         // SoA block convention: data rows, then 16-bit metadata records
};

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// n bytes (n even, <= 16) from a 2-byte aligned address, LSB-first into words.
template <int N>
__device__ __forceinline__ void ld_bytes(const uint8_t* p, uint32_t w[(N + 3) / 4]) {
#pragma unroll
  for (int i = 0; i < (N + 3) / 4; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) w[i / 2] |= ld_u16(p + 2 * i) << (16 * (i % 2));
}

// B-bit field i of an LSB-first bit stream held in words.
template <int B>
__device__ __forceinline__ uint32_t field(const uint32_t* w, int i) {
  const int p = B * i, k = p >> 5, s = p & 31;
  uint32_t v = w[k] >> s;
  if (s + B > 32) v |= w[k + 1] << (32 - s);
  return v & ((1u << B) - 1u);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16 consecutive outputs of one lane, rounded to nearest even in the output
// type (pairs through the packed converts, v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32).
template <int OUT>
__device__ __forceinline__ void store16(void* base, int64_t elem, const float x[kDpl]) {
  if constexpr (OUT == TQ_F32) {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  } else {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x2 p = {x[2 * i], x[2 * i + 1]};
      if constexpr (OUT == TQ_F16)
        h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
      else
        h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    uint4* q = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem);
    q[0] = make_uint4(h[0], h[1], h[2], h[3]);
    q[1] = make_uint4(h[4], h[5], h[6], h[7]);
  }
}

// Raw fields of one slot for this lane: its key bytes (or FP8 key bytes),
// the key norm, its value-code bytes, the value scale and zero.
template <int KEY_FP8, int KB, int VB>
struct SlotFields {
  static constexpr int kKeyBytes = KEY_FP8 ? kDpl : kDpl * KB / 8;
  static constexpr int kValBytes = kDpl * VB / 8;
  uint32_t kw[(kKeyBytes + 3) / 4 + 1];
  uint32_t vw[(kValBytes + 3) / 4 + 1];
  uint32_t gamma, scale_zero;
};

// kp / vp: the row's key data and value codes; gp: its key norm (MSE keys);
// sp: its value scale, the zero 2 bytes on.
template <int KEY_FP8, int KB, int VB, int VLM>
__device__ __forceinline__ void load_fields(const uint8_t* kp, const uint8_t* vp, const uint8_t* gp,
                                            const uint8_t* sp, int sub, SlotFields<KEY_FP8, KB, VB>& f) {
  using F = SlotFields<KEY_FP8, KB, VB>;
  f.kw[(F::kKeyBytes + 3) / 4] = 0u;
  f.vw[(F::kValBytes + 3) / 4] = 0u;
  ld_bytes<F::kKeyBytes>(kp + F::kKeyBytes * sub, f.kw);
  ld_bytes<F::kValBytes>(vp + F::kValBytes * sub, f.vw);
  f.gamma = KEY_FP8 ? 0u : ld_u16(gp);
  // Lloyd-Max values: sp is their norm, the only field
  f.scale_zero = VLM ? ld_u16(sp) : (ld_u16(sp) | (ld_u16(sp + 2) << 16));
}

// Each wave takes kGroups groups of 64 / (D / 16) consecutive rows (D / 16
// lanes per row); the loads of all its groups are issued before any is decoded, so a
// wave keeps several slots' worth of reads in flight.  The MSE presets, with
// more arithmetic per slot, take 4; FP8 keys keep 1 and more waves resident.
template <int KEY_FP8>
constexpr int groups_per_wave() { return KEY_FP8 ? 1 : 4; }

// VLM: Lloyd-Max values, decoded like MSE keys with the value codebook (which
// follows the key codebook in the table).
template <int D, int KEY_FP8, int KB, int VB, int VLM, int OUT>
__global__ __launch_bounds__(kThreads) void tq_dequant_kernel(DequantArgs a) {
  constexpr int kGroups = groups_per_wave<KEY_FP8 && !VLM>();
  constexpr int kLpr = D / kDpl;  // lanes per row
  constexpr int kRowsPerWave = 64 / kLpr;
  constexpr int kL = 1 << KB, kLv = 1 << VB;
  __shared__ float cent[KEY_FP8 ? 1 : kL];
  __shared__ float vcent[VLM ? kLv : 1];
  if (!KEY_FP8 || VLM) {
    if (!KEY_FP8 && threadIdx.x < kL) cent[threadIdx.x] = a.centroids[threadIdx.x];
    if (VLM && threadIdx.x < kLv) vcent[threadIdx.x] = a.centroids[(KEY_FP8 ? 0 : kL) + threadIdx.x];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (kLpr - 1);
  const uint32_t base = (blockIdx.x * kWaves + wave) * (kRowsPerWave * kGroups) + lane / kLpr;

  SlotFields<KEY_FP8, KB, VB> f[kGroups];
  uint32_t rows[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const uint32_t row0 = base + g * kRowsPerWave;
    const uint32_t row = row0 < static_cast<uint32_t>(a.num_rows) ? row0 : a.num_rows - 1;  // in bounds
    rows[g] = row0;
    const uint32_t t = row / static_cast<uint32_t>(a.num_kv_heads);
    const int h = static_cast<int>(row - t * a.num_kv_heads);
    const int64_t blk = a.block_table[t / static_cast<uint32_t>(a.block_size)];
    const uint32_t tb = t % static_cast<uint32_t>(a.block_size);
    constexpr int kKdata = KEY_FP8 ? D : D * KB / 8;
    constexpr int kKps = KEY_FP8 ? D : kKdata + 2;
    constexpr int kVdata = D * VB / 8;
    if (a.soa) {
      // SoA: row r = t * Hk + h of the block: [key data | value codes] at
      // r * kDb, then the fields (norm, scale, zero / scale, zero) at
      // 2 * (r * kNf + f) after the data region
      constexpr int kDb = kKdata + kVdata, kNf = (KEY_FP8 ? 0 : 1) + (VLM ? 1 : 2);
      const int64_t rows = static_cast<int64_t>(a.block_size) * a.num_kv_heads;
      const uint8_t* blkp = a.cache + blk * rows * a.slot_bytes;
      const int64_t r = static_cast<int64_t>(tb) * a.num_kv_heads + h;
      const uint8_t* drow = blkp + r * kDb;
      const uint8_t* rec = blkp + rows * kDb + r * (2 * kNf);
      load_fields<KEY_FP8, KB, VB, VLM>(drow, drow + kKdata, rec, rec + (KEY_FP8 ? 0 : 2), sub, f[g]);
    } else {
      const uint8_t* slot = a.cache + ((blk * a.block_size + tb) * a.num_kv_heads + h) * a.slot_bytes;
      load_fields<KEY_FP8, KB, VB, VLM>(slot, slot + kKps, slot + kKdata, slot + kKps + kVdata, sub, f[g]);
    }
  }

  float sg[kDpl];  // signs * (+-1/sqrt(D)), the lane sign of the butterflies undone
  if (!KEY_FP8 || VLM) {
    constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.0625f;
    const float c = tq::wht_lane_negated(sub) ? -kInvSqrtD : kInvSqrtD;
    const float4* sp = reinterpret_cast<const float4*>(a.signs + kDpl * sub);
#pragma unroll
    for (int i = 0; i < kDpl / 4; ++i) {
      const float4 s4 = sp[i];
      sg[4 * i] = s4.x * c;
      sg[4 * i + 1] = s4.y * c;
      sg[4 * i + 2] = s4.z * c;
      sg[4 * i + 3] = s4.w * c;
    }
  }

#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    // ---------------- key ----------------
    float k[kDpl];
    if (KEY_FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(f[g].kw[i], false);  // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(f[g].kw[i], true);   // bytes 2, 3
        k[4 * i] = lo[0];
        k[4 * i + 1] = lo[1];
        k[4 * i + 2] = hi[0];
        k[4 * i + 3] = hi[1];
      }
    } else {
      // rotated coordinates gamma * c[code], then s .* (H y) / sqrt(D) with the
      // store's butterflies
      const float gamma = __half2float(__ushort_as_half(static_cast<unsigned short>(f[g].gamma)));
#pragma unroll
      for (int i = 0; i < kDpl; ++i) k[i] = gamma * cent[field<KB>(f[g].kw, i)];
      tq::wht_inlane(k, 1);
      tq::wht_crosslane<kLpr>(k, sub);
#pragma unroll
      for (int i = 0; i < kDpl; ++i) k[i] *= sg[i];
    }
    // ---------------- value ----------------
    float v[kDpl];
    if (VLM) {  // as the keys: gamma_v * c_v[code], rotated back
      const float gv = __half2float(__ushort_as_half(static_cast<unsigned short>(f[g].scale_zero)));
#pragma unroll
      for (int i = 0; i < kDpl; ++i) v[i] = gv * vcent[field<VB>(f[g].vw, i)];
      tq::wht_inlane(v, 1);
      tq::wht_crosslane<kLpr>(v, sub);
#pragma unroll
      for (int i = 0; i < kDpl; ++i) v[i] *= sg[i];
    } else {
      const float sc = __half2float(__ushort_as_half(static_cast<unsigned short>(f[g].scale_zero & 0xFFFFu)));
      const float z = __half2float(__ushort_as_half(static_cast<unsigned short>(f[g].scale_zero >> 16)));
#pragma unroll
      for (int i = 0; i < kDpl; ++i) v[i] = fmaf(sc, static_cast<float>(field<VB>(f[g].vw, i)), z);  // exact product
    }

    if (rows[g] < static_cast<uint32_t>(a.num_rows)) {
      const uint32_t t = rows[g] / static_cast<uint32_t>(a.num_kv_heads);
      const int h = static_cast<int>(rows[g] - t * a.num_kv_heads);
      const int64_t e = static_cast<int64_t>(t) * a.out_tok_stride + h * D + kDpl * sub;
      store16<OUT>(a.key_out, e, k);
      store16<OUT>(a.value_out, e, v);
    }
  }
}

template <int D, int KEY_FP8, int KB, int VB, int VLM = 0>
int launch_dequant(const DequantArgs& a, int32_t out_dtype, hipStream_t stream) {
  const int64_t per_block = static_cast<int64_t>(kThreads / (D / kDpl)) * groups_per_wave<KEY_FP8 && !VLM>();
  const int blocks = static_cast<int>((a.num_rows + per_block - 1) / per_block);
  DequantArgs arg = a;
  void* args[] = {&arg};
  const void* fn =
      out_dtype == TQ_F32   ? reinterpret_cast<const void*>(&tq_dequant_kernel<D, KEY_FP8, KB, VB, VLM, TQ_F32>)
      : out_dtype == TQ_F16 ? reinterpret_cast<const void*>(&tq_dequant_kernel<D, KEY_FP8, KB, VB, VLM, TQ_F16>)
                            : reinterpret_cast<const void*>(&tq_dequant_kernel<D, KEY_FP8, KB, VB, VLM, TQ_BF16>);
  return tq::hip_status(hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args, 0, stream));
}

template <int D>
int launch_preset(int32_t preset, const DequantArgs& a, int32_t out_dtype, hipStream_t s) {
  switch (preset) {
    case TQ_K8V4: return launch_dequant<D, 1, 8, 4>(a, out_dtype, s);
    case TQ_4BIT_NC: return launch_dequant<D, 0, 4, 4>(a, out_dtype, s);
    case TQ_K3V4_NC: return launch_dequant<D, 0, 3, 4>(a, out_dtype, s);
    case TQ_3BIT_NC: return launch_dequant<D, 0, 3, 3>(a, out_dtype, s);
    case TQ_K8V3: return launch_dequant<D, 1, 8, 3>(a, out_dtype, s);
    case TQ_K4V3_NC: return launch_dequant<D, 0, 4, 3>(a, out_dtype, s);
    case TQ_2BIT_NC: return launch_dequant<D, 0, 2, 2>(a, out_dtype, s);
    case TQ_K8V3LM: return launch_dequant<D, 1, 8, 3, 1>(a, out_dtype, s);
    case TQ_3BIT_LM: return launch_dequant<D, 0, 3, 3, 1>(a, out_dtype, s);
    case TQ_K8V4LM: return launch_dequant<D, 1, 8, 4, 1>(a, out_dtype, s);
    case TQ_4BIT_LM: return launch_dequant<D, 0, 4, 4, 1>(a, out_dtype, s);
    case TQ_2BIT_LM: return launch_dequant<D, 0, 2, 2, 1>(a, out_dtype, s);
  }
  return TQ_EPRESET;
}

}  // namespace

extern "C" int tq_dequant_kv(const tq_layout* layout, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                             int32_t num_kv_heads, const int32_t* block_table, int32_t num_tokens, const float* signs,
                             const float* centroids, void* key_out, void* value_out, int32_t out_dtype,
                             int64_t out_tok_stride, void* stream) {
  int st = tq::validate_dequant(layout, kv_cache, num_blocks, block_size, num_kv_heads, block_table, num_tokens, signs,
                                centroids, key_out, value_out, out_dtype, out_tok_stride);
  if (st != TQ_OK || num_tokens == 0) return st;
  DequantArgs a;
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.signs = signs;
  a.centroids = centroids;
  a.key_out = key_out;
  a.value_out = value_out;
  a.out_tok_stride = out_tok_stride;
  a.num_rows = num_tokens * num_kv_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.slot_bytes = layout->slot_size_aligned;
  a.soa = layout->block_layout == TQ_LAYOUT_SOA;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layout->head_dim == 256 ? launch_preset<256>(layout->preset, a, out_dtype, s)
                                 : launch_preset<128>(layout->preset, a, out_dtype, s);
}
