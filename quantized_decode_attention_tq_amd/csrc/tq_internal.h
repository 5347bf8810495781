// Internal declarations shared by the host code and the launchers of libtq.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

// Records the HIP error of a failed launch for tq_last_hip_error() (per
// thread) and maps it to a status.
int hip_status(int hip_error);

inline bool block_size_ok(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// true when *L equals what tq_layout_init produces for (L->preset, L->head_dim)
bool layout_consistent(const tq_layout* L);

// stage-1 partials (B, Hq, S, D+1) fp32, rounded up to 256 bytes
size_t workspace_bytes(int64_t batch, int64_t num_q_heads, int64_t head_dim, int64_t num_kv_splits);

int validate_store(const tq_layout* L, const void* key, const void* value, int32_t in_dtype, int64_t num_tokens,
                   int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride, const int64_t* slot_mapping,
                   const void* kv_cache, int64_t num_blocks, int32_t block_size, const float* signs,
                   const float* centroids, const float* boundaries);

int validate_decode(const tq_layout* L, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                    const float* signs, const float* centroids, int32_t num_kv_splits, const void* workspace,
                    size_t ws_bytes);

int validate_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                    const void* workspace, size_t ws_bytes, const void* out, int32_t out_dtype);

// KV heads per stage-1 workgroup (one wave each) for this layout, or 0 when
// no grouping keeps every staged 16-byte chunk aligned.  A workgroup stages
// the 16 token rows of a tile restricted to its G heads: with G == Hk that
// is one contiguous run; otherwise every row piece (G * slot bytes at a row
// stride of Hk * slot) must start on a 16-byte boundary.
inline int decode_heads_per_wg(const tq_layout* L, int32_t num_kv_heads) {
  const int slot = L->slot_size_aligned;
  if (num_kv_heads <= 8) return num_kv_heads;
  if ((num_kv_heads * slot) % 16 != 0) return 0;
  for (int g = 8; g >= 1; g >>= 1)
    if (num_kv_heads % g == 0 && (g * slot) % 16 == 0) return g;
  return 0;
}

}  // namespace tq
