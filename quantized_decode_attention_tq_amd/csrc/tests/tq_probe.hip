// Probe kernels for the tests only (not part of libtq): each runs a single
// compiler builtin or bit helper so that a test can compare the GPU's lane
// layout / rounding with a host model.  All launches are one small block on
// the current device, synchronous, with every index inside the buffers the
// caller sized: n items, fixed per-item strides.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_bits.h"
#include "tq_wave.h"

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kBitsIn = 12, kBitsOut = 8;

// One helper call: inputs in[0..11], outputs out[0..7].
TQ_HD void run_bits_op(int op, const uint32_t* in, uint32_t* out) {
  for (int i = 0; i < kBitsOut; ++i) out[i] = 0;
  switch (op) {
    case 0: out[0] = tq::perm32(in[0], in[1], in[2]); break;
    case 1: out[0] = tq::alignbyte(in[0], in[1], in[2]); break;
    case 2: tq::key3_selectors(in[0], in[1], in[2], out); break;
    case 3: tq::lut8(in[0], tq::Lut8{in[1], in[2], in[3], in[4]}, out[0], out[1]); break;
    case 4: tq::lut16(in[0], tq::Lut8{in[1], in[2], in[3], in[4]}, tq::Lut8{in[5], in[6], in[7], in[8]}, out[0], out[1]); break;
    case 5: tq::val4_pairs(in[0], in[1], out); break;
    case 6: tq::val3_pairs(in[0], in[1], out); break;
    case 8: tq::val2_pairs(in[0], in[1], out); break;
    case 9:
      for (int k = 0; k < 4; ++k) out[k] = tq::key2_selector(in[0], k);
      break;
    case 10: tq::lm_value_selectors(in, out); break;
    case 14: tq::lm4_value_selectors(in, out); break;
    case 15: tq::lm2_value_selectors(in, out); break;
    case 11:  // pair fields 8 in[3] .. 8 in[3] + 7 of the stream in[0..2]
      for (int k = 0; k < 8; ++k) out[k] = tq::key3_pair_field(in[0], in[1], in[2], 8 * (in[3] & 1u) + k);
      break;
    case 13:  // windows of pair fields 8 in[3] .. 8 in[3] + 7
      for (int k = 0; k < 8; ++k) out[k] = tq::key3_pair_window(in[0], in[1], in[2], 8 * (in[3] & 1u) + k);
      break;
    case 12: {  // pair-table entries in[8] .. in[8] + 7 of the fp16 codebook in[0..7] (low halves)
      uint16_t h[8];
      for (int k = 0; k < 8; ++k) h[k] = static_cast<uint16_t>(in[k]);
      for (int k = 0; k < 8; ++k) out[k] = tq::key3_pair_entry(h, static_cast<int>((in[8] + k) & 63u));
      break;
    }
    case 7: {
      float f;
      uint32_t u = in[0];
      __builtin_memcpy(&f, &u, 4);
      out[0] = tq::f32_to_e4m3(f);
      break;
    }
    default: break;
  }
}

__global__ void bits_kernel(int op, const uint32_t* in, uint32_t* out, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    run_bits_op(op, in + static_cast<int64_t>(i) * kBitsIn, out + static_cast<int64_t>(i) * kBitsOut);
}

// a, b: per lane 4 dwords (8 halves); d: per lane 4 floats
__global__ void mfma32_kernel(const uint32_t* a, const uint32_t* b, float* d) {
  const int l = threadIdx.x;
  u32x4 av = {a[4 * l], a[4 * l + 1], a[4 * l + 2], a[4 * l + 3]};
  u32x4 bv = {b[4 * l], b[4 * l + 1], b[4 * l + 2], b[4 * l + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), __builtin_bit_cast(half8, bv), acc, 0, 0, 0);
  for (int i = 0; i < 4; ++i) d[4 * l + i] = acc[i];
}

// a, b: per lane 2 dwords (4 halves); d: per lane 4 floats
__global__ void mfma16_kernel(const uint32_t* a, const uint32_t* b, float* d) {
  const int l = threadIdx.x;
  u32x2 av = {a[2 * l], a[2 * l + 1]};
  u32x2 bv = {b[2 * l], b[2 * l + 1]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4, av), __builtin_bit_cast(half4, bv), acc, 0, 0, 0);
  for (int i = 0; i < 4; ++i) d[4 * l + i] = acc[i];
}

// FP8 (E4M3) -> fp16 pairs: out[2i] = bytes 0,1 of in[i]; out[2i+1] = bytes 2,3
__global__ void cvt_fp8_kernel(const uint32_t* in, uint32_t* out, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(in[i], 1.0f, false));
    out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(in[i], 1.0f, true));
  }
}

// Streaming read, the ceiling the decode's cache read is compared with:
// workgroup i reads the contiguous 16-byte chunks [i * chunk16, (i + 1) *
// chunk16) of the buffer with non-temporal loads, four in flight per lane;
// the xor of everything read decides a store that never happens, so no load
// is dead.  (64 KB per workgroup measured fastest on the MI355X: 6.25 TB/s on
// 205 MB, 6.7 TB/s on 1 GB; 256 KB and 1 MB pieces were 12-28% slower on 205 MB.)
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ in, int64_t chunk16,
                                                          int64_t n16, uint32_t* __restrict__ out) {
  uint32_t x = 0;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * chunk16;
  const int64_t e = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < e; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(in + i);
    const u32x4 b = __builtin_nontemporal_load(in + i + 256);
    const u32x4 c = __builtin_nontemporal_load(in + i + 512);
    const u32x4 d = __builtin_nontemporal_load(in + i + 768);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < e; i += 256) {
    const u32x4 a = __builtin_nontemporal_load(in + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) out[blockIdx.x] = x;
}

// The decode's reads without its arithmetic: the tiles of all sequences in
// order (a tile is 16 consecutive token rows of row16 16-byte chunks inside
// one cache block, found through the block table; sequence b holds tiles
// prefix[b] .. prefix[b + 1] - 1 of the list), split evenly over the
// workgroups whatever the mix of lengths, 16-byte non-temporal loads, two
// tiles at a time.  Wave w of a workgroup writes the XOR of the 32-bit
// words it read to out[4 * blockIdx.x + w] (so a test can check the bytes
// covered).
__global__ __launch_bounds__(256) void gather_read_kernel(const u32x4* __restrict__ cache,
                                                          const int32_t* __restrict__ block_table, int bt_stride,
                                                          const int32_t* __restrict__ prefix, int batch,
                                                          int block_size, int64_t row16, uint32_t* __restrict__ out) {
  const int64_t T = prefix[batch];
  const int t0 = static_cast<int>(T * blockIdx.x / gridDim.x);
  const int t1 = static_cast<int>(T * (blockIdx.x + 1) / gridDim.x);
  const int64_t tile16 = 16 * row16, blk16 = static_cast<int64_t>(block_size) * row16;
  int b = 0;  // sequence of tile t0: the last b with prefix[b] <= t0
  for (int lo = 0, hi = batch - 1; lo <= hi;) {
    const int mid = (lo + hi) / 2;
    if (prefix[mid] <= t0) {
      b = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  // base of list tile t (t >= the tile last passed to it)
  auto tile_base = [&](int t) {
    while (prefix[b + 1] <= t) ++b;
    const int j = t - prefix[b];  // tile of sequence b
    const int32_t blk = block_table[static_cast<int64_t>(b) * bt_stride + (j * 16) / block_size];
    return cache + static_cast<int64_t>(blk) * blk16 + static_cast<int64_t>((j * 16) % block_size) * row16;
  };
  uint32_t x = 0;
  int t = t0;
  for (; t + 1 < t1; t += 2) {
    const u32x4* p0 = tile_base(t);
    const u32x4* p1 = tile_base(t + 1);
#pragma unroll 2
    for (int64_t j = threadIdx.x; j < tile16; j += 256) {
      const u32x4 a = __builtin_nontemporal_load(p0 + j);
      const u32x4 c = __builtin_nontemporal_load(p1 + j);
      x ^= a.x ^ a.y ^ a.z ^ a.w ^ c.x ^ c.y ^ c.z ^ c.w;
    }
  }
  if (t < t1) {
    const u32x4* p0 = tile_base(t);
    for (int64_t j = threadIdx.x; j < tile16; j += 256) {
      const u32x4 a = __builtin_nontemporal_load(p0 + j);
      x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), m, 64));
  if ((threadIdx.x & 63) == 0) out[4 * blockIdx.x + (threadIdx.x >> 6)] = x;
}

// Plain copy of n16 16-byte chunks.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                   int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[i] = in[i];
}

// FP8 E4M3 encodes of fp32 inputs: out[3i] = the software encoder
// (tq::f32_to_e4m3), out[3i+1] = v_cvt_pk_fp8_f32, out[3i+2] =
// v_cvt_scalef32_pk_fp8_f32 with scale 1 (low byte of each).
typedef short v2i16 __attribute__((ext_vector_type(2)));
__global__ void fp8enc_kernel(const uint32_t* in, uint32_t* out, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float x = __uint_as_float(in[i]);
    out[3 * i] = tq::f32_to_e4m3(x);
    out[3 * i + 1] = __builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xFFu;
    const v2i16 old = {0, 0};
    out[3 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, x, x, 1.0f, false)) & 0xFFu;
  }
}

// one wave64: out[0..63], out[64..127] = the two results of permlane16_swap
// (v, v); out[128..191], out[192..255] = those of permlane32_swap (v, v)
__global__ void permlane_kernel(const uint32_t* in, uint32_t* out) {
  const int l = threadIdx.x;
  const uint32_t v = in[l];
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  out[l] = a[0];
  out[64 + l] = a[1];
  out[128 + l] = c[0];
  out[192 + l] = c[1];
}

// one wave64 per 64 inputs: out[0..63], [64..127], [128..191] = the wave
// sum, the wave maximum and the inclusive prefix sum of the wave's inputs
// as each lane holds them (the decode's work search builds on these)
__global__ void wave_ops_kernel(const int32_t* in, int32_t* out) {
  const int l = threadIdx.x;
  const int v = in[64 * blockIdx.x + l];
  int32_t* o = out + 192 * blockIdx.x;
  o[l] = tq::wave_sum_i(v);
  o[64 + l] = tq::wave_max_i(v);
  o[128 + l] = tq::wave_incl_scan_i(v);
}

int finish() {
  if (hipGetLastError() != hipSuccess) return -8;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -8;
}

}  // namespace

extern "C" {

// host model of the bit helpers (emulated byte permutes)
int tq_probe_bits_host(int op, const uint32_t* in, uint32_t* out, int n) {
  for (int i = 0; i < n; ++i) run_bits_op(op, in + static_cast<int64_t>(i) * kBitsIn, out + static_cast<int64_t>(i) * kBitsOut);
  return 0;
}

// same helpers on the GPU; in: device [n][12], out: device [n][8]
int tq_probe_bits_device(int op, const uint32_t* in, uint32_t* out, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(bits_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, 0, op, in, out, n);
  return finish();
}

// one wave64: a, b device [64][4] dwords, d device [64][4] floats
int tq_probe_mfma_16x16x32_f16(const uint32_t* a, const uint32_t* b, float* d) {
  hipLaunchKernelGGL(mfma32_kernel, dim3(1), dim3(64), 0, 0, a, b, d);
  return finish();
}

// one wave64: a, b device [64][2] dwords, d device [64][4] floats
int tq_probe_mfma_16x16x16_f16(const uint32_t* a, const uint32_t* b, float* d) {
  hipLaunchKernelGGL(mfma16_kernel, dim3(1), dim3(64), 0, 0, a, b, d);
  return finish();
}

// waves wave64s: in device [64 * waves] int32, out device [192 * waves] int32
int tq_probe_wave_ops(const int32_t* in, int32_t* out, int waves) {
  if (waves <= 0) return -1;
  hipLaunchKernelGGL(wave_ops_kernel, dim3(waves), dim3(64), 0, 0, in, out);
  return finish();
}

// one wave64: in device [64] dwords, out device [256] dwords
int tq_probe_permlane_swap(const uint32_t* in, uint32_t* out) {
  hipLaunchKernelGGL(permlane_kernel, dim3(1), dim3(64), 0, 0, in, out);
  return finish();
}

// in: device [n] fp32 bits; out: device [3n] (software, cvt_pk, cvt_scalef32)
int tq_probe_fp8_encode(const uint32_t* in, uint32_t* out, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fp8enc_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, 0, in, out, n);
  return finish();
}

// in: device [n] dwords of 4 FP8 bytes; out: device [2n] fp16 pairs
int tq_probe_cvt_fp8_f16(const uint32_t* in, uint32_t* out, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(cvt_fp8_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, 0, in, out, n);
  return finish();
}

// Streaming read of bytes (multiple of 16) from a device buffer in pieces
// of chunk bytes (a multiple of 16) per workgroup; out: device uint32 with at
// least ceil(bytes / chunk) entries (written only in a case that does not
// occur); asynchronous on `stream` (timed by the caller).
int tq_probe_stream_read(const void* in, int64_t bytes, int64_t chunk, uint32_t* out, void* stream) {
  if (bytes <= 0 || chunk <= 0 || bytes % 16 || chunk % 16) return -1;
  const int64_t blocks = (bytes + chunk - 1) / chunk;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(in), chunk / 16, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

// The decode's tile reads of a paged cache (row_bytes: bytes of one token
// row, all KV heads, a multiple of 16; prefix: device int32 [batch + 1],
// prefix[b] = tiles of sequences 0 .. b - 1) by `groups` workgroups; out:
// device uint32 [4 * groups].  Asynchronous on `stream`.
int tq_probe_gather_read(const void* cache, const int32_t* block_table, int bt_stride, const int32_t* prefix,
                         int batch, int block_size, int64_t row_bytes, int groups, uint32_t* out, void* stream) {
  if (batch <= 0 || groups <= 0 || row_bytes <= 0 || row_bytes % 16 || block_size < 16 || block_size % 16)
    return -1;
  hipLaunchKernelGGL(gather_read_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(cache), block_table, bt_stride,
                     prefix, batch, block_size, row_bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

// Copy bytes (multiple of 16), asynchronous on `stream`.
int tq_probe_copy(const void* in, void* out, int64_t bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(in), static_cast<u32x4*>(out), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
