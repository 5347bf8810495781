// Internal declarations shared by the host code and the launchers of libtq.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

// Records the HIP error of a failed launch for tq_last_hip_error() (per
// thread) and maps it to a status.
int hip_status(int hip_error);

// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes) the first time
// fn is launched on the current device (cached per (kernel, device) under a
// lock; later calls return TQ_OK at once).  TQ_EUNSUPPORTED if fn declares
// static LDS: the stage-1 kernels place a table at LDS address 0.
int set_max_lds_once(const void* fn, int bytes);

inline bool block_size_ok(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// true when *L equals what tq_layout_init produces for (L->preset, L->head_dim)
bool layout_consistent(const tq_layout* L);

// decode workspace: sequence table + partial rows (layout below), rounded up to 256 bytes
size_t workspace_bytes(int64_t batch, int64_t num_q_heads, int64_t head_dim, int64_t num_kv_splits);

int validate_store(const tq_layout* L, const void* key, const void* value, int32_t in_dtype, int64_t num_tokens,
                   int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride, const int64_t* slot_mapping,
                   const void* kv_cache, int64_t num_blocks, int32_t block_size, const float* signs,
                   const float* centroids, const float* boundaries);

int validate_decode(const tq_layout* L, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                    const float* signs, const float* centroids, int32_t num_kv_splits, int32_t sliding_window,
                    float value_gate, const void* workspace, size_t ws_bytes);

int validate_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                    const void* workspace, size_t ws_bytes, const void* out, int32_t out_dtype);

int validate_dequant(const tq_layout* L, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                     int32_t num_kv_heads, const int32_t* block_table, int32_t num_tokens, const float* signs,
                     const float* centroids, const void* key_out, const void* value_out, int32_t out_dtype,
                     int64_t out_tok_stride);

// ---- decode workspace and stage-1 launch plan ----
//
// Stage 1 cuts the batch into U "units" of work: the tiles (16 tokens) of
// each sequence are split into S_b ranges so that every unit holds about the
// same number of tiles (sum_b S_b <= U), whatever the mix of lengths.  U =
// batch * S_int, where S_int >= the caller's num_kv_splits S is raised until
// the grid has about kTargetWorkgroups workgroups (two per compute unit of an
// MI355X).  The workspace holds
//   [table]  int32 [batch][2] = (first unit, number of units) of each sequence
//   [rows]   fp32 [U][Hq][kPartPad + head_dim]: the normalized partial output
//            of a (unit, query head) followed by its natural-log LSE (padded
//            to 16-byte rows).
constexpr int64_t kTargetWorkgroups = 512;
// SoA tile images: bytes of padding after each image row of data (G data rows)
constexpr int kSoaRowPad = 16;
// The raise of S_int stops where a unit of the longest possible sequence
// would hold fewer tiles than this: a unit's fixed cost (work search, query
// rotation, ring fill) needs a few tiles to amortize.
constexpr int64_t kMinTilesPerUnit = 16;
constexpr int64_t kPartPad = 4;  // LSE + 3 pad floats after the head_dim outputs
// 3-bit MSE keys decode through a 64-entry table of fp16 centroid pairs in
// LDS (two dims per lookup), one copy per lane of the wave so that the 64
// lanes' reads never share a bank: 64 entries x 64 copies x 4 bytes at the
// start of a stage-1 workgroup's dynamic LDS, ahead of the ring.
constexpr int kKey3LutCopies = 64;
constexpr int kKey3LutBytes = 64 * kKey3LutCopies * 4;
inline size_t key_lut_bytes(const tq_layout* L) {
  return (!L->key_fp8 && L->key_bits == 3) ? static_cast<size_t>(kKey3LutBytes) : 0;
}

inline int64_t table_bytes(int64_t batch) { return (8 * batch + 255) / 256 * 256; }

// Largest S_int any launch with this (batch, S) uses (the plan's raise
// assumes at least one workgroup per unit).
inline int64_t max_splits(int64_t batch, int64_t num_splits) {
  if (batch <= 0) return num_splits;
  const int64_t per = batch * num_splits;
  const int64_t m = (kTargetWorkgroups + per - 1) / per;
  return num_splits * (m > 1 ? m : 1);
}

// Launch plan of decode stage 1 (host).  A workgroup serves G KV heads with
// P waves each (P <= 2, G * P <= 8 waves).  G = Hk when Hk <= 8, so a tile of the
// group is one contiguous run of cache rows; otherwise the largest divisor
// of Hk (<= 8) whose row pieces stay 16-byte aligned.  The P waves of a head
// split its tiles.  A tile image (16 token rows of the group) takes spt 1 KB
// slots of LDS; the ring holds R super-tiles of P tiles (two-deep unless a
// super-tile is small), sized for two
// workgroups per compute unit (after the 3-bit key table, if any).  max_tiles: tiles of the longest possible
// sequence (block-table width), which caps S_int.
struct DecodePlan {
  int G, P, R, spt, contiguous;
  int dslots;      // SoA: slots of a tile image's data part (0 for combined slots)
  int soa_pad;     // SoA: pad bytes after each 16-token image row of data (a multiple of 16)
  int tpw;         // tiles each wave computes per super-tile (between barriers)
  size_t lds;      // dynamic LDS bytes per workgroup
  int64_t units;   // U
  int64_t grid;    // workgroups = U * (Hk / G) * head groups
};

// Direct-to-LDS loads (1 KB each) a stage-1 wave issues per tile: at most
// this many for any head count (a wave of G waves per tile takes ceil(spt /
// G) of the tile's spt loads).  head_dim 128: slots of 196 / 134 / 118 / 102
// / 180 / 118 / 70 / 178 / 100 / 194 / 132 / 68 bytes in preset order; SoA images pad each
// image row by 16 bytes and round the data part and the metadata part up to
// whole slots separately, which takes one load more with one KV head for
// k8v4, 4bit_nc, 3bit_nc and 2bit_nc (and their Lloyd-Max-value twins).
// head_dim 256: slots of 388 / 262 / 230 / 198 / 356 / 230 / 134 / 354 / 196
// / 386 / 260 / 132 bytes.
constexpr int max_dma_loads(int preset, bool soa = false, int head_dim = 128) {
  const bool d256 = head_dim == 256;
  switch (preset) {
    case TQ_K8V4: return d256 ? (soa ? 8 : 7) : (soa ? 5 : 4);
    case TQ_4BIT_NC: return d256 ? (soa ? 6 : 5) : (soa ? 4 : 3);
    case TQ_K3V4_NC: return d256 ? (soa ? 5 : 4) : 3;
    case TQ_3BIT_NC: return d256 ? (soa ? 5 : 4) : (soa ? 3 : 2);
    case TQ_K8V3: return d256 ? (soa ? 7 : 6) : 4;
    case TQ_K4V3_NC: return d256 ? (soa ? 5 : 4) : 3;
    case TQ_2BIT_NC: return d256 ? (soa ? 4 : 3) : (soa ? 3 : 2);
    case TQ_K8V3LM: return d256 ? (soa ? 7 : 6) : 4;
    case TQ_3BIT_LM: return d256 ? (soa ? 5 : 4) : (soa ? 3 : 2);
    case TQ_K8V4LM: return d256 ? (soa ? 8 : 7) : (soa ? 5 : 4);
    case TQ_4BIT_LM: return d256 ? (soa ? 6 : 5) : (soa ? 4 : 3);
    case TQ_2BIT_LM: return d256 ? (soa ? 4 : 3) : (soa ? 3 : 2);
  }
  return 0;
}

inline int decode_plan(const tq_layout* L, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t num_splits, int64_t max_tiles, DecodePlan* p) {
  constexpr size_t kLdsBudget = 52 * 1024, kLdsMax = 160 * 1024;  // two-deep rings measured best
  const int64_t slot = L->slot_size_aligned;
  const int64_t row = num_kv_heads * slot;
  const int group = num_q_heads / num_kv_heads;
  const int64_t hgroups = (group + 15) / 16;
  const bool soa = L->block_layout == TQ_LAYOUT_SOA;
  int G = 0;
  if (soa) {
    // SoA pieces must stay 16-byte multiples: all KV heads, or 8 of them
    if (num_kv_heads > 8 && num_kv_heads % 8 != 0) return TQ_EUNSUPPORTED;
    G = num_kv_heads <= 8 ? num_kv_heads : 8;
  } else if (num_kv_heads <= 8) {
    G = num_kv_heads;
  } else {
    for (int d = 8; d >= 1 && G == 0; --d)
      if (num_kv_heads % d == 0 && (d * slot) % 16 == 0 && row % 16 == 0) G = d;
    for (int d = 8; d >= 1 && G == 0; --d)
      if (num_kv_heads % d == 0) G = d;
  }
  // At most 2 phase waves per head: with few KV heads, smaller workgroups
  // and rings let more of them share a CU.  Against 8 / G phases, stage 1
  // on 205 MB of cache took 26-29% less time with 1 KV head (4-8 phases
  // before), 9% less on 3bit_nc with 2 (k8v4 unchanged), and 22-30% less
  // at head_dim 256 with 2 KV heads; 1 phase was no better than 4.
  const int P = G >= 8 ? 1 : (8 / G < 2 ? 8 / G : 2);
  const bool contiguous = G == num_kv_heads;
  const int64_t wg_per_unit = (num_kv_heads / G) * hgroups;
  const int64_t per = static_cast<int64_t>(batch) * num_splits * wg_per_unit;
  int64_t s_int = num_splits * (per > 0 && per < kTargetWorkgroups ? (kTargetWorkgroups + per - 1) / per : 1);
  const int64_t cap_p = (max_tiles + P - 1) / P;  // more units than P-tile steps per sequence are idle
  const int64_t cap_t = (max_tiles + kMinTilesPerUnit - 1) / kMinTilesPerUnit;
  const int64_t cap = cap_p < cap_t ? cap_p : cap_t;
  if (s_int > num_splits && s_int > cap) s_int = cap > num_splits ? cap : num_splits;
  const int64_t piece = G * slot;
  const int64_t tc_max = contiguous ? row : 16 * ((piece + 30) / 16);  // chunks per tile image
  // SoA: 16 image rows of G * (key data + value data) bytes plus a 16-byte
  // pad, then 16 x G records of 2 * fields bytes, each part in whole 1 KB
  // slots
  const int64_t soa_data = L->soa_data_bytes, soa_meta = 2 * static_cast<int64_t>(L->soa_meta_fields);
  const int dslots = soa ? static_cast<int>((G * soa_data + kSoaRowPad + 63) / 64) : 0;
  const int spt = soa ? dslots + static_cast<int>((G * soa_meta + 63) / 64) : static_cast<int>((tc_max + 63) / 64);
  // MSE keys: two tiles per wave between barriers (two independent chains
  // to interleave), when the ring still fits two workgroups per CU (never
  // at head_dim 256, whose tile images are twice as large)
  const int tpw =
      (!L->key_fp8 && L->head_dim == 128 && 2 * static_cast<size_t>(P) * spt * 1024 * 2 <= 80 * 1024) ? 2 : 1;
  const size_t entry = static_cast<size_t>(P) * tpw * spt * 1024;
  size_t R = kLdsBudget / entry;
  R = R < 2 ? 2 : (R > 4 ? 4 : R);
  // phase merge: per (phase > 0, head) a lane's outputs (32 per 128-dim
  // half) and its LSE
  const size_t merge = P > 1 ? static_cast<size_t>(P - 1) * G * (32 * (L->head_dim / 128) + 1) * 64 * 4 : 0;
  p->G = G;
  p->P = P;
  p->R = static_cast<int>(R);
  p->tpw = tpw;
  p->spt = spt;
  p->contiguous = contiguous;
  p->dslots = dslots;
  p->soa_pad = soa ? kSoaRowPad : 0;
  p->lds = key_lut_bytes(L) + (R * entry > merge ? R * entry : merge);
  p->units = static_cast<int64_t>(batch) * s_int;
  p->grid = p->units * wg_per_unit;
  const int loads = (spt + G - 1) / G;  // DMA slots per wave per tile of its phase
  const int64_t blk_bytes = 128 * row;  // largest block (block_size 128)
  if (p->lds > kLdsMax || loads > max_dma_loads(L->preset, soa, L->head_dim) || p->grid > 0x7FFFFFFF || p->units > 0x7FFFFFFF ||
      blk_bytes > 0xFFFFFFFFLL || s_int > max_splits(batch, num_splits))
    return TQ_EUNSUPPORTED;
  return TQ_OK;
}

}  // namespace tq
