// tq_store: quantize new K/V rows and write their combined slots into the
// paged cache, one fused launch ([PR] "实现拆解" item 4: bucketing, norm,
// index packing and value quantization in one kernel; [API] _store_kv).
//
// Work mapping (gfx950, wave64): a "row" is one (token, KV head) pair.  Each
// wave owns 8 rows, 8 lanes per row, 16 contiguous dims per lane (D = 128).
// The randomized Hadamard rotation runs in registers: the butterfly strides
// 1..8 are inside a lane, strides 16/32/64 are lane exchanges within the
// row's 8-lane group ([TQ+] "Background": random signs, then the WHT).
// Norms and min/max reduce over the same 8 lanes.  The codebook and its
// boundaries sit in LDS.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "tq.h"
#include "tq_bits.h"
#include "tq_internal.h"

namespace {

constexpr int kD = 128;
constexpr int kDpl = 16;           // dims per lane
constexpr int kRowsPerWave = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kMaxSlot = 208;  // >= every preset's slot at head_dim 128, 16-byte multiple

struct StoreArgs {
  const uint16_t* key;
  const uint16_t* value;
  int64_t num_rows;  // N * Hk
  int64_t key_tok_stride;
  int64_t val_tok_stride;
  const int64_t* slot_mapping;
  uint8_t* cache;
  const float* signs;
  const float* centroids;
  const float* boundaries;
  int32_t num_kv_heads;
  int32_t slot_bytes;  // slot_size_aligned
  int32_t is_bf16;
};

__device__ __forceinline__ float widen16(uint32_t bits, bool bf16) {
  if (bf16) return __uint_as_float(bits << 16);
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

// Value of lane (l ^ m) for m = 1, 2, 4 (within each 8-lane row group), by
// DPP lane moves: no LDS round trip.  xor 1 / xor 2 are quad permutes; xor 4
// is the quad reversal (l ^ 3) followed by the half-row mirror (l ^ 7).
__device__ __forceinline__ float xor_shfl(float v, int m) {
  int x = __float_as_int(v);
  if (m == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if (m == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else {
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  }
  return __int_as_float(x);
}

__device__ __forceinline__ void load_row16(const uint16_t* p, bool bf16, float x[kDpl]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = widen16(w[i] & 0xFFFFu, bf16);
    x[2 * i + 1] = widen16(w[i] >> 16, bf16);
  }
}

__device__ __forceinline__ void st16(uint8_t* p, uint32_t v) { *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v); }

// count of boundaries strictly below u, binary search over the sorted table
template <int KB>
__device__ __forceinline__ int bucketize(float u, const float* __restrict__ b_lds) {
  constexpr int L = 1 << KB;
  int i = 0;
#pragma unroll
  for (int step = L / 2; step >= 1; step >>= 1) i += (u > b_lds[i + step - 1]) ? step : 0;
  return i;
}

template <int KEY_FP8, int KB, int VB, int NC>
__global__ __launch_bounds__(kThreads) void tq_store_kernel(StoreArgs a) {
  __shared__ float c_lds[16];
  __shared__ float b_lds[16];
  if (!KEY_FP8) {
    if (threadIdx.x < (1 << KB)) c_lds[threadIdx.x] = a.centroids[threadIdx.x];
    if (threadIdx.x < (1 << KB) - 1) b_lds[threadIdx.x] = a.boundaries[threadIdx.x];
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 7;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * kRowsPerWave + (lane >> 3);
  const bool active = row0 < a.num_rows;
  const int64_t row = active ? row0 : a.num_rows - 1;  // inactive rows compute on a valid row, store nothing
  const int64_t n = row / a.num_kv_heads;
  const int h = static_cast<int>(row - n * a.num_kv_heads);
  const bool bf16 = a.is_bf16 != 0;

  float x[kDpl], v[kDpl];
  load_row16(a.key + n * a.key_tok_stride + h * kD + sub * kDpl, bf16, x);
  load_row16(a.value + n * a.val_tok_stride + h * kD + sub * kDpl, bf16, v);

  const int64_t m = a.slot_mapping[n];
  uint8_t* slot = a.cache + (m * a.num_kv_heads + h) * static_cast<int64_t>(a.slot_bytes);
  const bool write = active && m >= 0;

  // ---------------- key ----------------
  constexpr int kKeyBytesPerLane = KEY_FP8 ? kDpl : (kDpl * KB) / 8;
  uint32_t kbytes[kDpl / 2] = {};  // lane's key bytes, little-endian, packed 4 per dword
  uint32_t gamma_bits = 0;
  if (KEY_FP8) {
    // Hardware convert (round to nearest even) after clamping to the E4M3
    // range, which gives the saturating encoder's bytes for every non-NaN
    // input; a wave holding a NaN key takes the software encoder.
    bool has_nan = false;
#pragma unroll
    for (int i = 0; i < kDpl; ++i) has_nan |= __builtin_isnan(x[i]);
    if (__any(has_nan)) {
#pragma unroll
      for (int i = 0; i < kDpl; ++i) kbytes[i / 4] |= tq::f32_to_e4m3(x[i]) << (8 * (i % 4));
    } else {
#pragma unroll
      for (int j = 0; j < kDpl / 4; ++j) {
        uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x[4 * j], -448.f, 448.f),
                                                     __builtin_amdgcn_fmed3f(x[4 * j + 1], -448.f, 448.f), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x[4 * j + 2], -448.f, 448.f),
                                            __builtin_amdgcn_fmed3f(x[4 * j + 3], -448.f, 448.f), w, true);
        kbytes[j] = w;
      }
    }
  } else {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kDpl; ++i) ss = fmaf(x[i], x[i], ss);
    ss += xor_shfl(ss, 1);
    ss += xor_shfl(ss, 2);
    ss += xor_shfl(ss, 4);
    const float nu = sqrtf(ss);

    float y[kDpl];
    const float4* sg = reinterpret_cast<const float4*>(a.signs + sub * kDpl);
#pragma unroll
    for (int i = 0; i < kDpl / 4; ++i) {
      float4 s4 = sg[i];
      y[4 * i + 0] = x[4 * i + 0] * s4.x;
      y[4 * i + 1] = x[4 * i + 1] * s4.y;
      y[4 * i + 2] = x[4 * i + 2] * s4.z;
      y[4 * i + 3] = x[4 * i + 3] * s4.w;
    }
    // Walsh-Hadamard butterflies, natural (Sylvester) order
#pragma unroll
    for (int hs = 1; hs < kDpl; hs <<= 1) {
#pragma unroll
      for (int i = 0; i < kDpl; ++i) {
        if ((i & hs) == 0) {
          float p = y[i], q = y[i + hs];
          y[i] = p + q;
          y[i + hs] = p - q;
        }
      }
    }
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) {
      const bool upper = (sub & msk) != 0;
#pragma unroll
      for (int i = 0; i < kDpl; ++i) {
        float o = xor_shfl(y[i], msk);
        y[i] = upper ? (o - y[i]) : (y[i] + o);
      }
    }
    // u = (H s.*x) / (sqrt(D) * nu); nu == 0 gives u = 0 and a zero norm field
    const float inv = nu > 0.f ? 1.0f / (nu * 11.313708498984761f) : 0.f;
    float cs = 0.f;
    int code[kDpl];
#pragma unroll
    for (int i = 0; i < kDpl; ++i) {
      code[i] = bucketize<KB>(y[i] * inv, b_lds);
      const float c = c_lds[code[i]];
      cs = fmaf(c, c, cs);
    }
    cs += xor_shfl(cs, 1);
    cs += xor_shfl(cs, 2);
    cs += xor_shfl(cs, 4);
    float gamma = nu;
    if (NC) gamma = nu > 0.f ? nu / sqrtf(cs) : 0.f;
    gamma_bits = __half_as_ushort(__float2half_rn(gamma));
    // LSB-first bit stream: code i of the lane at bit KB*i of the lane's chunk
    uint64_t bitsacc = 0;
#pragma unroll
    for (int i = 0; i < kDpl; ++i) bitsacc |= static_cast<uint64_t>(code[i]) << (KB * i);
#pragma unroll
    for (int i = 0; i < kDpl / 2; ++i) kbytes[i] = 0;
    kbytes[0] = static_cast<uint32_t>(bitsacc);
    kbytes[1] = static_cast<uint32_t>(bitsacc >> 32);
  }

  // ---------------- value ----------------
  float vmin = v[0], vmax = v[0];
#pragma unroll
  for (int i = 1; i < kDpl; ++i) {
    vmin = fminf(vmin, v[i]);
    vmax = fmaxf(vmax, v[i]);
  }
#pragma unroll
  for (int msk = 1; msk < 8; msk <<= 1) {
    vmin = fminf(vmin, xor_shfl(vmin, msk));
    vmax = fmaxf(vmax, xor_shfl(vmax, msk));
  }
  constexpr int kLevels = (1 << VB) - 1;
  const __half z16 = __float2half_rn(vmin);
  const float s32 = __fdiv_rn(__fsub_rn(vmax, vmin), static_cast<float>(kLevels));
  const __half s16 = __float2half_rn(s32);
  const float zf = __half2float(z16);
  const float sf = __half2float(s16);
  uint64_t vacc = 0;
  if (sf != 0.f) {
    const float inv = __fdiv_rn(1.0f, sf);
#pragma unroll
    for (int i = 0; i < kDpl; ++i) {
      float r = __fadd_rn(__fmul_rn(__fsub_rn(v[i], zf), inv), 0.5f);
      r = fminf(fmaxf(floorf(r), 0.f), static_cast<float>(kLevels));  // NaN -> 0
      vacc |= static_cast<uint64_t>(static_cast<uint32_t>(r)) << (VB * i);
    }
  }
  constexpr int kValBytesPerLane = (kDpl * VB) / 8;

  // ---------------- stores ----------------
  const int kdata = KEY_FP8 ? kD : (kD * KB) / 8;
  const int kps = KEY_FP8 ? kD : kdata + 2;
  const int vdata = (kD * VB) / 8;
  if (a.num_kv_heads % kRowsPerWave == 0) {
    // The wave's 8 rows are 8 consecutive heads of one token: 8 adjacent
    // slots, 16-byte aligned.  Assemble them in LDS, then write them with
    // 16-byte stores.
    __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][kRowsPerWave * kMaxSlot];
    uint8_t* sl = stage[wave] + (lane >> 3) * a.slot_bytes;
    uint8_t* kp = sl + sub * kKeyBytesPerLane;
#pragma unroll
    for (int i = 0; i < kKeyBytesPerLane / 2; ++i) st16(kp + 2 * i, kbytes[i / 2] >> (16 * (i % 2)));
    if (!KEY_FP8 && sub == 0) st16(sl + kdata, gamma_bits);
    uint8_t* vp = sl + kps + sub * kValBytesPerLane;
#pragma unroll
    for (int i = 0; i < kValBytesPerLane / 2; ++i) st16(vp + 2 * i, static_cast<uint32_t>(vacc >> (16 * i)));
    if (sub == 0) {
      st16(sl + kps + vdata, __half_as_ushort(s16));
      st16(sl + kps + vdata + 2, __half_as_ushort(z16));
    }
    __syncthreads();
    // every row of the wave has the same token, activity and slot mapping
    if (write) {
      uint8_t* dst = slot - (lane >> 3) * static_cast<int64_t>(a.slot_bytes);  // slot of the wave's first head
      const int nchunk = (kRowsPerWave * a.slot_bytes) >> 4;
      for (int c = lane; c < nchunk; c += 64)
        *reinterpret_cast<uint4*>(dst + 16 * c) = *reinterpret_cast<const uint4*>(stage[wave] + 16 * c);
    }
  } else if (write) {
    uint8_t* kp = slot + sub * kKeyBytesPerLane;
#pragma unroll
    for (int i = 0; i < kKeyBytesPerLane / 2; ++i) st16(kp + 2 * i, kbytes[i / 2] >> (16 * (i % 2)));
    if (!KEY_FP8 && sub == 0) st16(slot + kdata, gamma_bits);
    uint8_t* vp = slot + kps + sub * kValBytesPerLane;
#pragma unroll
    for (int i = 0; i < kValBytesPerLane / 2; ++i) st16(vp + 2 * i, static_cast<uint32_t>(vacc >> (16 * i)));
    if (sub == 0) {
      st16(slot + kps + vdata, __half_as_ushort(s16));
      st16(slot + kps + vdata + 2, __half_as_ushort(z16));
    }
  }
}

template <int KEY_FP8, int KB, int VB, int NC>
int launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return TQ_EINVAL;
  StoreArgs arg = a;
  void* args[] = {&arg};
  return tq::hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&tq_store_kernel<KEY_FP8, KB, VB, NC>),
                                        dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args, 0, stream));
}

}  // namespace

extern "C" int tq_store(const tq_layout* layout, const void* key, const void* value, int32_t in_dtype,
                        int64_t num_tokens, int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride,
                        const int64_t* slot_mapping, void* kv_cache, int64_t num_blocks, int32_t block_size,
                        const float* signs, const float* centroids, const float* boundaries, void* stream) {
  int st = tq::validate_store(layout, key, value, in_dtype, num_tokens, num_kv_heads, key_tok_stride, val_tok_stride,
                              slot_mapping, kv_cache, num_blocks, block_size, signs, centroids, boundaries);
  if (st != TQ_OK || num_tokens == 0) return st;
  StoreArgs a;
  a.key = static_cast<const uint16_t*>(key);
  a.value = static_cast<const uint16_t*>(value);
  a.num_rows = num_tokens * num_kv_heads;
  a.key_tok_stride = key_tok_stride;
  a.val_tok_stride = val_tok_stride;
  a.slot_mapping = slot_mapping;
  a.cache = static_cast<uint8_t*>(kv_cache);
  a.signs = signs;
  a.centroids = centroids;
  a.boundaries = boundaries;
  a.num_kv_heads = num_kv_heads;
  a.slot_bytes = layout->slot_size_aligned;
  a.is_bf16 = in_dtype == TQ_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (layout->preset) {
    case TQ_K8V4: return launch_store<1, 8, 4, 0>(a, s);
    case TQ_4BIT_NC: return launch_store<0, 4, 4, 1>(a, s);
    case TQ_K3V4_NC: return launch_store<0, 3, 4, 1>(a, s);
    case TQ_3BIT_NC: return launch_store<0, 3, 3, 1>(a, s);
  }
  return TQ_EPRESET;
}
