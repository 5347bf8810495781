// Walsh-Hadamard butterflies over a D-vector (D = 128 or 256) held by D / 16
// consecutive lanes of a wave, 16 consecutive coordinates per lane (lane sub
// = lane % (D / 16) holds coordinates 16*sub .. 16*sub + 15), natural
// (Sylvester) order.  Strides 1..8 are inside a lane; strides 16, 32, 64
// (and 128) pair lane l with lane l ^ 1, 2, 4 (and 8) of its group through
// DPP lane moves (no LDS).  Shared by the store (the forward rotation) and
// the dequant (its transpose).
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

constexpr int kWhtPerLane = 16;

// Value of lane (l ^ m) for m = 1, 2, 4, 8 (within each 16-lane row).  xor 1
// / xor 2 are quad permutes; xor 4 is the quad reversal (l ^ 3) followed by
// the half-row mirror (l ^ 7); xor 8 is the row rotation by 8.
__device__ __forceinline__ float xor_shfl(float v, int m) {
  int x = __float_as_int(v);
  if (m == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if (m == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else if (m == 4) {
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  } else {
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8
  }
  return __int_as_float(x);
}

// In-lane butterflies of strides first_stride .. 8: (p, q) -> (p + q, p - q).
__device__ __forceinline__ void wht_inlane(float y[kWhtPerLane], int first_stride) {
#pragma unroll
  for (int hs = 1; hs < kWhtPerLane; hs <<= 1) {
    if (hs < first_stride) continue;
#pragma unroll
    for (int i = 0; i < kWhtPerLane; ++i) {
      if ((i & hs) == 0) {
        const float p = y[i], q = y[i + hs];
        y[i] = p + q;
        y[i + hs] = p - q;
      }
    }
  }
}

// Strides 16 .. 8 * LANES (LANES = D / 16 lanes per vector): the lower lane of a pair takes p + q, the upper one
// p - q.  Each lane keeps its coordinates times a lane sign sigma (equal on
// both lanes of a pair before the stride): w <- w + e * w_partner with e = -1
// on the upper lane and +1 on the lower one gives sigma*(p+q) on the lower
// lane and -sigma*(p-q) on the upper one, so each stride is one fma per value
// and flips sigma on the upper lanes.  On return the lane holds its
// transform coordinates times wht_lane_sign(sub).
template <int LANES>
__device__ __forceinline__ void wht_crosslane(float y[kWhtPerLane], int sub) {
#pragma unroll
  for (int msk = 1; msk < LANES; msk <<= 1) {
    const float e = (sub & msk) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < kWhtPerLane; ++i) y[i] = fmaf(xor_shfl(y[i], msk), e, y[i]);
  }
}

// The sign wht_crosslane leaves on lane sub's coordinates: (-1)^popcount(sub).
__device__ __forceinline__ bool wht_lane_negated(int sub) { return (__builtin_popcount(sub) & 1) != 0; }

}  // namespace tq
