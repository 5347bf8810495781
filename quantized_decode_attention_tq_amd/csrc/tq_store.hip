// tq_store: quantize new K/V rows and write their combined slots into the
// paged cache, one fused launch ([PR] "实现拆解" item 4: bucketing, norm,
// index packing and value quantization in one kernel; [API] _store_kv).
//
// Work mapping (gfx950, wave64): a "row" is one (token, KV head) pair, held
// by D / 16 lanes (8 at head_dim 128, 16 at 256), 16 contiguous dims per
// lane; a wave owns 64 / (D / 16) rows.  The randomized Hadamard rotation
// runs in registers: the butterfly strides 1..8 are inside a lane, strides
// 16 .. D / 2 are lane exchanges within the row's lane group ([TQ+]
// "Background": random signs, then the WHT).  Norms and min/max reduce over
// the same lanes.  The codebook and its boundaries sit in LDS.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "tq.h"
#include "tq_bits.h"
#include "tq_internal.h"
#include "tq_wht.h"

namespace {

using tq::xor_shfl;

constexpr int kDpl = 16;           // dims per lane
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStageRows = 8;  // rows assembled per 16-byte-store group
// Rows of a workgroup at head_dim D (D / 16 lanes per row).
template <int D>
constexpr int rows_per_block() { return kThreads / (D / kDpl); }
// >= every preset's slot at head_dim D, 16-byte multiple
template <int D>
constexpr int max_slot() { return D == 128 ? 208 : 400; }

struct StoreArgs {
  const uint16_t* key;
  const uint16_t* value;
  int32_t num_rows;  // tokens of this launch * Hk, below 2^31
  int64_t key_tok_stride;
  int64_t val_tok_stride;
  const int64_t* slot_mapping;
  uint8_t* cache;
  const float* signs;
  const float* centroids;
  const float* boundaries;
  int32_t num_kv_heads;
  int32_t slot_bytes;  // slot_size_aligned
  int32_t soa;         // SoA block convention: data rows, then 16-bit metadata records
  int32_t bs_log2;     // log2(block_size) (SoA addressing)
};

// 16 consecutive bf16 / fp16 elements -> fp32
template <int BF16>
__device__ __forceinline__ void load_row16(const uint16_t* p, float x[kDpl]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (BF16) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    } else {
      x[2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
      x[2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
    }
  }
}

__device__ __forceinline__ void st16(uint8_t* p, uint32_t v) { *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v); }

// Bucket search over the sorted boundaries, kept in LDS in breadth-first
// (Eytzinger) order: node n (1 .. 2^KB - 1) holds the boundary the plain
// binary search probes after taking the branches spelled by the bits of n
// below its leading one.  The walk n <- 2n + (u > tree[n]) ends on node
// 2^KB + #{boundaries < u}.  The walk carries 4n, the node's byte offset.
template <int KB>
__device__ __forceinline__ uint32_t tree_search(float u, const float* __restrict__ tree) {
  uint32_t m = 4;
#pragma unroll
  for (int d = 0; d < KB; ++d) {
    const float t = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(tree) + m);
    m = 2 * m + (u > t ? 4u : 0u);
  }
  return m;
}

// Sum, mod 2^32, of the 2^KB terms that the search's end nodes carry into
// word k of a lane's packed key bits (codes that straddle into the next word
// carry none).
template <int KB>
__host__ __device__ constexpr uint32_t key_bias(int k) {
  uint32_t r = 0;
  for (int i = 0; i < kDpl; ++i) {
    const int p = KB * i;
    if ((p >> 5) == k && (p & 31) + KB < 32) r += 1u << ((p & 31) + KB);
  }
  return r;
}

// Packs B-bit fields LSB-first into 32-bit words: field i at bit B*i.
template <int B>
struct Pack32 {
  uint32_t w[2] = {0u, 0u};
  // m = 4 * the search's end node 2^B + code: added whole, the 2^B terms
  // are removed once per word by finish_nodes()
  __device__ __forceinline__ void add_node(int i, uint32_t m) {
    const int p = B * i, k = p >> 5, s = p & 31;
    w[k] += s >= 2 ? m << (s - 2) : m >> (2 - s);
    if (s + B > 32) w[k + 1] += __builtin_amdgcn_ubfe(m, 34 - s, s + B - 32);
  }
  __device__ __forceinline__ void finish_nodes() {
    w[0] -= key_bias<B>(0);
    w[1] -= key_bias<B>(1);
  }
  __device__ __forceinline__ void or_code(int i, uint32_t c) {
    const int p = B * i, k = p >> 5, s = p & 31;
    w[k] |= c << s;
    if (s + B > 32) w[k + 1] |= c >> (32 - s);
  }
};

// Lloyd-Max quantization of one row held by LPR = D / 16 lanes (16 coordinates each):
// norm, randomized Hadamard rotation in registers, bucket search over the
// LDS boundary tree, packed codes and the fp16 norm field (norm-corrected
// when NC_).  Used for MSE keys and for Lloyd-Max values alike ([TQ+]
// "What landed": values take the keys' rotation and codebook).
template <int B, int NC_, int LPR>
__device__ __forceinline__ void mse_quantize(const float x[kDpl], const float* __restrict__ signs, int sub,
                                             const float* tree, const float* cent, uint32_t out[2],
                                             uint32_t& gamma_bits) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kDpl; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
  for (int msk = 1; msk < LPR; msk <<= 1) ss += xor_shfl(ss, msk);
  const float nu = sqrtf(ss);

  // Walsh-Hadamard butterflies, natural (Sylvester) order.  Stride 1 takes
  // the signs in: with s = +-1, s_i x_i is exact, so fma(x_i, s_i, +-s_j x_j)
  // rounds exactly as the sum of the signed pair does.
  float y[kDpl];
  const float4* sg = reinterpret_cast<const float4*>(signs + sub * kDpl);
#pragma unroll
  for (int i = 0; i < kDpl / 4; ++i) {
    const float4 s4 = sg[i];
    const float q0 = x[4 * i + 1] * s4.y, q1 = x[4 * i + 3] * s4.w;
    y[4 * i + 0] = fmaf(x[4 * i], s4.x, q0);
    y[4 * i + 1] = fmaf(x[4 * i], s4.x, -q0);
    y[4 * i + 2] = fmaf(x[4 * i + 2], s4.z, q1);
    y[4 * i + 3] = fmaf(x[4 * i + 2], s4.z, -q1);
  }
  tq::wht_inlane(y, 2);
  // strides 16 .. D / 2 across the row's lanes; the lane sign they leave is
  // folded into the scale below
  tq::wht_crosslane<LPR>(y, sub);
  // u = (H s.*x) / (sqrt(D) * nu); nu == 0 gives u = 0 and a zero norm field
  constexpr float kSqrtD = LPR == 8 ? 11.313708498984761f : 16.f;
  const float inv0 = nu > 0.f ? 1.0f / (nu * kSqrtD) : 0.f;
  const float inv = tq::wht_lane_negated(sub) ? -inv0 : inv0;
  float cs = 0.f;
  Pack32<B> kp;
#pragma unroll
  for (int i = 0; i < kDpl; ++i) {
    const uint32_t m4 = tree_search<B>(y[i] * inv, tree);
    const float c = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(cent) + m4);
    cs = fmaf(c, c, cs);
    kp.add_node(i, m4);
  }
  kp.finish_nodes();
  out[0] = kp.w[0];
  out[1] = kp.w[1];
#pragma unroll
  for (int msk = 1; msk < LPR; msk <<= 1) cs += xor_shfl(cs, msk);
  float gamma = nu;
  if (NC_) gamma = nu > 0.f ? nu / sqrtf(cs) : 0.f;
  gamma_bits = __half_as_ushort(__float2half_rn(gamma));
}

// The codebook of B bits at (centroids, boundaries) into LDS: the search tree
// of the boundaries in breadth-first order (node n = 1 .. 2^B - 1) and the
// centroids at 2^B + code (the end node of each search).
template <int B>
__device__ __forceinline__ void load_tables(const float* centroids, const float* boundaries, float* tree,
                                            float* cent) {
  constexpr int kL = 1 << B;
  const int t = threadIdx.x;
  if (t >= 1 && t < kL) {
    const int d = 31 - __builtin_clz(t);  // depth of node t
    const int p = t - (1 << d);           // branches taken to reach it
    tree[t] = boundaries[(p << (B - d)) + (1 << (B - d - 1)) - 1];
  }
  if (t < kL) cent[kL + t] = centroids[t];
}

// VLM: Lloyd-Max values (rotated, codebook after the key codebook in the
// tables, norm-corrected), else uniform min/max values.
template <int D, int KEY_FP8, int KB, int VB, int NC, int VLM, int BF16>
__global__ __launch_bounds__(kThreads) void tq_store_kernel(StoreArgs a) {
  constexpr int kLpr = D / kDpl;  // lanes per row
  constexpr int kRowsPerWave = 64 / kLpr;
  constexpr int kL = 1 << KB, kLv = 1 << VB;
  __shared__ float tree[KEY_FP8 ? 4 : kL];      // node 1 .. kL - 1: boundaries in search order
  __shared__ float cent[KEY_FP8 ? 8 : 2 * kL];  // kL + code: centroid of the search's end node
  __shared__ float vtree[VLM ? kLv : 1];
  __shared__ float vcent[VLM ? 2 * kLv : 1];
  if (!KEY_FP8 || VLM) {
    if (!KEY_FP8) load_tables<KB>(a.centroids, a.boundaries, tree, cent);
    if (VLM) {
      const int ko = KEY_FP8 ? 0 : kL;  // the value codebook follows the key codebook
      load_tables<VB>(a.centroids + ko, a.boundaries + (KEY_FP8 ? 0 : kL - 1), vtree, vcent);
    }
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (kLpr - 1);
  const uint32_t row0 = (blockIdx.x * kWaves + wave) * kRowsPerWave + lane / kLpr;
  const bool active = row0 < static_cast<uint32_t>(a.num_rows);
  const uint32_t row = active ? row0 : a.num_rows - 1;  // inactive rows compute on a valid row, store nothing
  const uint32_t n = row / static_cast<uint32_t>(a.num_kv_heads);
  const int h = static_cast<int>(row - n * a.num_kv_heads);

  float x[kDpl], v[kDpl];
  load_row16<BF16>(a.key + n * a.key_tok_stride + h * D + sub * kDpl, x);
  load_row16<BF16>(a.value + n * a.val_tok_stride + h * D + sub * kDpl, v);

  const int64_t m = a.slot_mapping[n];
  uint8_t* slot = a.cache + (m * a.num_kv_heads + h) * static_cast<int64_t>(a.slot_bytes);
  const bool write = active && m >= 0;
  // SoA ([API] _store_kv): row r = t * Hk + h of the block holds [key data |
  // value data] at r * kDb; its fields (norm, scale, zero / scale, zero)
  // follow the data region as 16-bit values at 2 * (r * kNf + f)
  constexpr int kDb = (KEY_FP8 ? D : D * KB / 8) + D * VB / 8;
  constexpr int kNf = (KEY_FP8 ? 0 : 1) + (VLM ? 1 : 2);
  const int64_t mm = m >= 0 ? m : 0;
  const int64_t blk_rows = static_cast<int64_t>(a.num_kv_heads) << a.bs_log2;  // rows of a block
  uint8_t* blkp = a.cache + (mm >> a.bs_log2) * blk_rows * a.slot_bytes;
  const int64_t r = (mm & ((int64_t{1} << a.bs_log2) - 1)) * a.num_kv_heads + h;
  uint8_t* drow = blkp + r * kDb;
  uint8_t* mrec = blkp + blk_rows * kDb + r * (2 * kNf);

  // ---------------- key ----------------
  constexpr int kKeyBytesPerLane = KEY_FP8 ? kDpl : (kDpl * KB) / 8;
  uint32_t kbytes[kDpl / 4] = {};  // lane's key bytes, little-endian, packed 4 per dword
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
    mse_quantize<(KEY_FP8 ? 2 : KB), NC, kLpr>(x, a.signs, sub, tree, cent, kbytes, gamma_bits);
  }

  // ---------------- value ----------------
  constexpr int kLevels = (1 << VB) - 1;
  Pack32<VB> vp32;
  __half z16 = __ushort_as_half(0), s16 = __ushort_as_half(0);  // uniform codes: zero, scale
  uint32_t vgamma_bits = 0;                                          // Lloyd-Max codes: norm
  if constexpr (VLM != 0) {
    mse_quantize<VB, 1, kLpr>(v, a.signs, sub, vtree, vcent, vp32.w, vgamma_bits);
  } else {
  float vmin = v[0], vmax = v[0];
#pragma unroll
  for (int i = 1; i < kDpl; ++i) {
    vmin = fminf(vmin, v[i]);
    vmax = fmaxf(vmax, v[i]);
  }
#pragma unroll
  for (int msk = 1; msk < kLpr; msk <<= 1) {
    vmin = fminf(vmin, xor_shfl(vmin, msk));
    vmax = fmaxf(vmax, xor_shfl(vmax, msk));
  }
  z16 = __float2half_rn(vmin);
  const float s32 = __fdiv_rn(__fsub_rn(vmax, vmin), static_cast<float>(kLevels));
  s16 = __float2half_rn(s32);
  const float zf = __half2float(z16);
  const float sf = __half2float(s16);
  if (sf != 0.f) {
    // code = floor((v - zero) / scale + 1/2), decided in fp32 through the
    // reciprocal of the scale, taken 2^-22 high: v, zero and scale are short
    // binary numbers, so quotients exactly at a half-integer are common, and
    // the raised reciprocal puts them strictly above it, rounding up as the
    // definition does.  A quotient within about x * 2^-21 below a
    // half-integer may round up as well (one step, next to the decision
    // boundary).
    const float inv = __fmul_rn(__fdiv_rn(1.0f, sf), 1.0f + 0x1p-22f);
#pragma unroll
    for (int i = 0; i < kDpl; ++i) {
      // fp32 roundings as written: no fused multiply-add here
#pragma clang fp contract(off)
      const float q = (v[i] - zf) * inv;
      float r = q + 0.5f;
      // clamp to [0, levels] (NaN -> 0), then truncate: floor of a
      // non-negative number
      r = fminf(fmaxf(r, 0.f), static_cast<float>(kLevels));
      vp32.or_code(i, static_cast<uint32_t>(r));
    }
  }
  }
  constexpr int kValBytesPerLane = (kDpl * VB) / 8;

  // ---------------- stores ----------------
  const int kdata = KEY_FP8 ? D : (D * KB) / 8;
  const int kps = KEY_FP8 ? D : kdata + 2;
  const int vdata = (D * VB) / 8;
  // the row's fields: key bytes, value bytes, norm, scale (zero 2 bytes on)
  auto put = [&](uint8_t* kp0, uint8_t* vp0, uint8_t* gp, uint8_t* sp) {
    uint8_t* kp = kp0 + sub * kKeyBytesPerLane;
#pragma unroll
    for (int i = 0; i < kKeyBytesPerLane / 2; ++i) st16(kp + 2 * i, kbytes[i / 2] >> (16 * (i % 2)));
    if (!KEY_FP8 && sub == 0) st16(gp, gamma_bits);
    uint8_t* vp = vp0 + sub * kValBytesPerLane;
#pragma unroll
    for (int i = 0; i < kValBytesPerLane / 2; ++i) st16(vp + 2 * i, vp32.w[i / 2] >> (16 * (i % 2)));
    if (sub == 0) {
      if (VLM) {
        st16(sp, vgamma_bits);
      } else {
        st16(sp, __half_as_ushort(s16));
        st16(sp + 2, __half_as_ushort(z16));
      }
    }
  };
  const int fs = KEY_FP8 ? 0 : 2;  // SoA: byte of the scale inside a record
  if (a.num_kv_heads % kStageRows == 0) {
    // Each group of 8 consecutive rows (one wave at head_dim 128, two at
    // 256) is 8 consecutive heads of one token: 8 adjacent slots (SoA: 8
    // adjacent data rows and 8 adjacent records), 16-byte aligned.  Assemble
    // them in LDS, then write them with 16-byte stores.
    constexpr int kGt = kStageRows * kLpr;  // threads of a group
    __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads / kGt][kStageRows * max_slot<D>()];
    const int gi = threadIdx.x / kGt, gt = threadIdx.x % kGt;
    const int q = gt / kLpr;  // row of the group
    if (a.soa) {
      uint8_t* sd = stage[gi] + q * kDb;
      uint8_t* sm = stage[gi] + kStageRows * kDb + q * (2 * kNf);
      put(sd, sd + kdata, sm, sm + fs);
    } else {
      uint8_t* sl = stage[gi] + q * a.slot_bytes;
      put(sl, sl + kps, sl + kdata, sl + kps + vdata);
    }
    __syncthreads();
    // every row of the group has the same token, activity and slot mapping
    if (write) {
      if (a.soa) {
        uint8_t* dd = drow - q * kDb;            // data row of the group's first head
        uint8_t* dm = mrec - q * (2 * kNf);      // its record
        constexpr int kDc = kStageRows * kDb / 16, kMc = kStageRows * 2 * kNf / 16;
        for (int c = gt; c < kDc + kMc; c += kGt) {
          uint8_t* dst = c < kDc ? dd + 16 * c : dm + 16 * (c - kDc);
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(stage[gi] + 16 * c);
        }
      } else {
        uint8_t* dst = slot - q * static_cast<int64_t>(a.slot_bytes);  // slot of the group's first head
        const int nchunk = (kStageRows * a.slot_bytes) >> 4;
        for (int c = gt; c < nchunk; c += kGt)
          *reinterpret_cast<uint4*>(dst + 16 * c) = *reinterpret_cast<const uint4*>(stage[gi] + 16 * c);
      }
    }
  } else if (write) {
    if (a.soa)
      put(drow, drow + kdata, mrec, mrec + fs);
    else
      put(slot, slot + kps, slot + kdata, slot + kps + vdata);
  }
}

template <int D, int KEY_FP8, int KB, int VB, int NC, int VLM = 0>
int launch_store(const StoreArgs& a, bool bf16, hipStream_t stream) {
  const int blocks = (a.num_rows + rows_per_block<D>() - 1) / rows_per_block<D>();
  StoreArgs arg = a;
  void* args[] = {&arg};
  const void* fn = bf16 ? reinterpret_cast<const void*>(&tq_store_kernel<D, KEY_FP8, KB, VB, NC, VLM, 1>)
                        : reinterpret_cast<const void*>(&tq_store_kernel<D, KEY_FP8, KB, VB, NC, VLM, 0>);
  return tq::hip_status(hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), args, 0, stream));
}

template <int D>
int launch_preset(int32_t preset, const StoreArgs& a, bool bf16, hipStream_t s) {
  switch (preset) {
    case TQ_K8V4: return launch_store<D, 1, 8, 4, 0>(a, bf16, s);
    case TQ_4BIT_NC: return launch_store<D, 0, 4, 4, 1>(a, bf16, s);
    case TQ_K3V4_NC: return launch_store<D, 0, 3, 4, 1>(a, bf16, s);
    case TQ_3BIT_NC: return launch_store<D, 0, 3, 3, 1>(a, bf16, s);
    case TQ_K8V3: return launch_store<D, 1, 8, 3, 0>(a, bf16, s);
    case TQ_K4V3_NC: return launch_store<D, 0, 4, 3, 1>(a, bf16, s);
    case TQ_2BIT_NC: return launch_store<D, 0, 2, 2, 1>(a, bf16, s);
    case TQ_K8V3LM: return launch_store<D, 1, 8, 3, 0, 1>(a, bf16, s);
    case TQ_3BIT_LM: return launch_store<D, 0, 3, 3, 1, 1>(a, bf16, s);
    case TQ_K8V4LM: return launch_store<D, 1, 8, 4, 0, 1>(a, bf16, s);
    case TQ_4BIT_LM: return launch_store<D, 0, 4, 4, 1, 1>(a, bf16, s);
    case TQ_2BIT_LM: return launch_store<D, 0, 2, 2, 1, 1>(a, bf16, s);
  }
  return TQ_EPRESET;
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
  a.num_kv_heads = num_kv_heads;
  a.key_tok_stride = key_tok_stride;
  a.val_tok_stride = val_tok_stride;
  a.cache = static_cast<uint8_t*>(kv_cache);
  a.signs = signs;
  a.centroids = centroids;
  a.boundaries = boundaries;
  a.slot_bytes = layout->slot_size_aligned;
  a.soa = layout->block_layout == TQ_LAYOUT_SOA;
  a.bs_log2 = 31 - __builtin_clz(static_cast<unsigned>(block_size));
  const bool bf16 = in_dtype == TQ_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the kernel indexes rows in 32 bits: launches of at most 2^30 rows
  const int64_t chunk = (int64_t{1} << 30) / num_kv_heads > 0 ? (int64_t{1} << 30) / num_kv_heads : 1;
  for (int64_t t0 = 0; t0 < num_tokens; t0 += chunk) {
    const int64_t nt = num_tokens - t0 < chunk ? num_tokens - t0 : chunk;
    a.key = static_cast<const uint16_t*>(key) + t0 * key_tok_stride;
    a.value = static_cast<const uint16_t*>(value) + t0 * val_tok_stride;
    a.slot_mapping = slot_mapping + t0;
    a.num_rows = static_cast<int32_t>(nt * num_kv_heads);
    st = layout->head_dim == 256 ? launch_preset<256>(layout->preset, a, bf16, s)
                                 : launch_preset<128>(layout->preset, a, bf16, s);
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}
