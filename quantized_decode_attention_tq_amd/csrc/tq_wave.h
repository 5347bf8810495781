// Whole-wave (64-lane) integer reductions and prefix sum for the decode's
// work search, built from DPP row operations and the gfx950 row swaps, so
// that no step goes through the LDS crossbar (a ds_bpermute per step, each
// a round trip of ~100 cycles, was most of the search's time).
//
// Lanes form 4 rows of 16.  Reductions: quad_perm xor 1 and xor 2 combine
// each quad, row_ror 4 and 8 the quads of a row, permlane16_swap and
// permlane32_swap (each lane receives its own value and that of lane l ^ 16,
// resp. l ^ 32, one in each result) the rows; every lane ends with the
// total.  Inclusive scan: row_shr 1, 2, 4, 8 (sources before the row's start
// read as 0) give each row its own prefix sums; row_bcast 15 adds the last
// lane of rows 0 and 2 to rows 1 and 3, row_bcast 31 that of row 1 to rows
// 2 and 3.
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

template <class Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror 8
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  v = op(static_cast<int>(a[0]), static_cast<int>(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  return op(static_cast<int>(c[0]), static_cast<int>(c[1]));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  return wave_reduce_i(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ int wave_max_i(int v) {
  return wave_reduce_i(v, [](int x, int y) { return x > y ? x : y; });
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr 1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr 4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr 8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast 15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast 31 into rows 2, 3
  return v;
}

}  // namespace tq
