// Host side of libtq: presets and slot layout, the Lloyd-Max codebook
// solvers, the Rademacher sign generator, workspace sizing and argument
// validation.  No device code and no HIP calls live here.
//
// Citations name the source page and section:
//   [PR]  prhub summary of vLLM PR #38479, "实现拆解" / "关键源码片段"
//   [API] vLLM API docs, vllm.v1.attention.backends.turboquant_attn
//   [TQ+] Atlas docs "TurboQuant+ -- KV-cache compression beyond the Google baseline"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "tq.h"
#include "tq_internal.h"

namespace {

struct PresetDef {
  const char* name;
  int key_fp8, key_bits, value_bits, norm_correction, value_lloyd_max;
};

// [PR] "实现拆解" item 1 (four named presets with key bits, value bits and
// norm correction); "评论区精华" (k8v4 means FP8 keys and 4-bit values).
// The rest follow [TQ+] "What landed": asymmetric pairs (FP8 or 4-bit keys
// over 3-bit values), the 2-bit codebook, and Lloyd-Max values (the keys'
// rotation and codebook family on the value rows) at 2, 3 and 4 bits, with
// this library's key and value codecs at those widths.
constexpr PresetDef kPresets[TQ_NUM_PRESETS] = {
    {"turboquant_k8v4", 1, 8, 4, 0, 0},
    {"turboquant_4bit_nc", 0, 4, 4, 1, 0},
    {"turboquant_k3v4_nc", 0, 3, 4, 1, 0},
    {"turboquant_3bit_nc", 0, 3, 3, 1, 0},
    {"turboquant_k8v3", 1, 8, 3, 0, 0},
    {"turboquant_k4v3_nc", 0, 4, 3, 1, 0},
    {"turboquant_2bit_nc", 0, 2, 2, 1, 0},
    {"turboquant_k8v3lm", 1, 8, 3, 0, 1},
    {"turboquant_3bit_lm", 0, 3, 3, 1, 1},
    {"turboquant_k8v4lm", 1, 8, 4, 0, 1},
    {"turboquant_4bit_lm", 0, 4, 4, 1, 1},
    {"turboquant_2bit_lm", 0, 2, 2, 1, 1},
};

}  // namespace

extern "C" const char* tq_version(void) { return "libtq 0.1 (gfx950)"; }

extern "C" const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument (null pointer, negative size or misaligned tensor)";
    case TQ_EPRESET: return "unknown preset";
    case TQ_EHEADDIM: return "unsupported head_dim (kernels support 128 and 256)";
    case TQ_EBLOCK: return "block_size must be 16, 32, 64 or 128";
    case TQ_EGQA: return "num_q_heads must be a positive multiple of num_kv_heads";
    case TQ_EWORKSPACE: return "workspace too small";
    case TQ_EDTYPE: return "unsupported element type";
    case TQ_EHIP: return "HIP launch failed";
    case TQ_EUNSUPPORTED: return "unsupported combination";
  }
  return "unknown status";
}

extern "C" int tq_preset_from_name(const char* name, int32_t* preset) {
  if (!name || !preset) return TQ_EINVAL;
  for (int i = 0; i < TQ_NUM_PRESETS; ++i) {
    if (std::strcmp(name, kPresets[i].name) == 0) {
      *preset = i;
      return TQ_OK;
    }
  }
  return TQ_EPRESET;
}

// [API] TurboQuantAttentionImpl.__init__: key bytes ceil(D*bits/8), or D for
// FP8 keys; value bytes ceil(D*value_bits/8).  [API] _continuation_prefill:
// the key region is larger than the code bytes (fp16 norm follows) and the
// value region ends with two 16-bit fields (scale, zero).  [PR]
// get_kv_cache_shape: slot rounded up to an even byte count.
extern "C" int tq_layout_init(int32_t preset, int32_t head_dim, tq_layout* out) {
  return tq_layout_init_ex(preset, head_dim, TQ_LAYOUT_AOS, out);
}

extern "C" int tq_layout_init_ex(int32_t preset, int32_t head_dim, int32_t block_layout, tq_layout* out) {
  if (!out || (block_layout != TQ_LAYOUT_AOS && block_layout != TQ_LAYOUT_SOA)) return TQ_EINVAL;
  if (preset < 0 || preset >= TQ_NUM_PRESETS) return TQ_EPRESET;
  if (head_dim <= 0 || head_dim % 8 != 0) return TQ_EHEADDIM;
  const PresetDef& p = kPresets[preset];
  tq_layout L{};
  L.preset = preset;
  L.head_dim = head_dim;
  L.key_fp8 = p.key_fp8;
  L.key_bits = p.key_bits;
  L.value_bits = p.value_bits;
  L.norm_correction = p.norm_correction;
  L.n_centroids = p.key_fp8 ? 0 : (1 << p.key_bits);
  L.key_data_bytes = p.key_fp8 ? head_dim : (head_dim * p.key_bits + 7) / 8;
  L.key_packed_size = p.key_fp8 ? head_dim : L.key_data_bytes + 2;
  L.value_data_bytes = (head_dim * p.value_bits + 7) / 8;
  L.value_lloyd_max = p.value_lloyd_max;
  L.value_packed_size = L.value_data_bytes + (p.value_lloyd_max ? 2 : 4);  // norm, or scale + zero
  L.slot_size = L.key_packed_size + L.value_packed_size;
  L.slot_size_aligned = (L.slot_size + 1) / 2 * 2;
  L.block_layout = block_layout;
  // SoA ([API] _continuation_prefill constants): the rows' data, then 16-bit
  // fields; the two regions fill the same block bytes as the slots (slot
  // sizes are even, so there is no padding to account for)
  L.soa_data_bytes = block_layout == TQ_LAYOUT_SOA ? L.key_data_bytes + L.value_data_bytes : 0;
  L.soa_meta_fields = block_layout == TQ_LAYOUT_SOA ? (p.key_fp8 ? 0 : 1) + (p.value_lloyd_max ? 1 : 2) : 0;
  if (block_layout == TQ_LAYOUT_SOA && L.soa_data_bytes + 2 * L.soa_meta_fields != L.slot_size_aligned)
    return TQ_EHEADDIM;
  *out = L;
  return TQ_OK;
}

namespace tq {

bool layout_consistent(const tq_layout* L) {
  if (!L) return false;
  tq_layout ref;
  if (tq_layout_init_ex(L->preset, L->head_dim, L->block_layout, &ref) != TQ_OK) return false;
  return std::memcmp(&ref, L, sizeof(tq_layout)) == 0;
}

}  // namespace tq

extern "C" int tq_kv_cache_shape(const tq_layout* layout, int64_t num_blocks, int32_t block_size,
                                 int32_t num_kv_heads, int64_t shape_out[4]) {
  if (!tq::layout_consistent(layout) || !shape_out || num_blocks < 0 || num_kv_heads <= 0) return TQ_EINVAL;
  if (!tq::block_size_ok(block_size)) return TQ_EBLOCK;
  shape_out[0] = num_blocks;
  shape_out[1] = block_size;
  shape_out[2] = num_kv_heads;
  shape_out[3] = layout->slot_size_aligned;
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook ([PR] "关键源码片段", centroids.py: Lloyd-Max conditions
// for the coordinate marginal N(0, 1/d) of a randomly rotated unit vector).
// ---------------------------------------------------------------------------

namespace {

constexpr double kInvSqrt2 = 0.70710678118654752440;
constexpr double kInvSqrt2Pi = 0.39894228040143267794;

double std_normal_pdf(double z) { return std::isinf(z) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * z * z); }

// P(a < Z < b) for Z ~ N(0,1), evaluated with erfc on the tail side so that
// far cells keep their relative precision.
double std_normal_mass(double a, double b) {
  if (a >= 0.0) {
    double ta = std::erfc(a * kInvSqrt2);
    double tb = std::isinf(b) ? 0.0 : std::erfc(b * kInvSqrt2);
    return 0.5 * (ta - tb);
  }
  if (b <= 0.0) {
    double tb = std::erfc(-b * kInvSqrt2);
    double ta = std::isinf(a) ? 0.0 : std::erfc(-a * kInvSqrt2);
    return 0.5 * (tb - ta);
  }
  double below_a = std::isinf(a) ? 0.0 : 0.5 * std::erfc(-a * kInvSqrt2);
  double above_b = std::isinf(b) ? 0.0 : 0.5 * std::erfc(b * kInvSqrt2);
  return 1.0 - below_a - above_b;
}

// Exact mode: the optimum for a symmetric density is antisymmetric, so the
// positive half (cells [0,t1), ..., [t_{h-1}, inf)) is iterated with the
// closed-form Gaussian cell mean (phi(a) - phi(b)) / (Phi(b) - Phi(a)) and
// mirrored.  Works in units of sigma; scaled by 1/sqrt(d) at the end.
std::vector<double> lloyd_max_exact(int d, int bits) {
  const int levels = 1 << bits, half = levels / 2;
  std::vector<double> p(half), t(half + 1), nxt(half);
  for (int k = 0; k < half; ++k) p[k] = (k + 0.5) * 3.0 / half;
  for (int it = 0; it < 200000; ++it) {
    t[0] = 0.0;
    for (int k = 1; k < half; ++k) t[k] = 0.5 * (p[k - 1] + p[k]);
    t[half] = std::numeric_limits<double>::infinity();
    double delta = 0.0;
    for (int k = 0; k < half; ++k) {
      nxt[k] = (std_normal_pdf(t[k]) - std_normal_pdf(t[k + 1])) / std_normal_mass(t[k], t[k + 1]);
      delta = std::fmax(delta, std::fabs(nxt[k] - p[k]));
    }
    p.swap(nxt);
    if (delta < 1e-15) break;
  }
  const double sigma = 1.0 / std::sqrt(static_cast<double>(d));
  std::vector<double> c(levels);
  for (int k = 0; k < half; ++k) {
    c[half + k] = p[k] * sigma;
    c[half - 1 - k] = -p[k] * sigma;
  }
  return c;
}

// The pages' solver: uniform start on +-3.5 sigma, midpoint boundaries, outer
// cells closed at +-10.5 sigma, trapezoid rule with 200 intervals for the
// zeroth and first moments, at most 200 rounds, and on convergence (no move
// >= 1e-10) the centroids from before that round are kept.
std::vector<double> lloyd_max_pages_trapz(int d, int bits) {
  const int levels = 1 << bits;
  const double var = 1.0 / d, sigma = std::sqrt(var);
  const double norm = 1.0 / std::sqrt(2.0 * M_PI * var);
  auto pdf = [&](double x) { return norm * std::exp(-x * x / (2.0 * var)); };
  auto trapz = [&](auto f, double a, double b) {
    const int n = 200;
    const double h = (b - a) / n;
    double s = 0.5 * (f(a) + f(b));
    for (int i = 1; i < n; ++i) s += f(a + i * h);
    return s * h;
  };
  const double lo = -3.5 * sigma, hi = 3.5 * sigma;
  std::vector<double> c(levels), edges(levels + 1), nxt(levels);
  for (int i = 0; i < levels; ++i) c[i] = lo + (hi - lo) * (i + 0.5) / levels;
  for (int it = 0; it < 200; ++it) {
    edges[0] = 3.0 * lo;
    for (int i = 1; i < levels; ++i) edges[i] = 0.5 * (c[i - 1] + c[i]);
    edges[levels] = 3.0 * hi;
    double delta = 0.0;
    for (int i = 0; i < levels; ++i) {
      double a = edges[i], b = edges[i + 1];
      double num = trapz([&](double x) { return x * pdf(x); }, a, b);
      double den = trapz(pdf, a, b);
      nxt[i] = den > 1e-15 ? num / den : c[i];
      delta = std::fmax(delta, std::fabs(nxt[i] - c[i]));
    }
    if (delta < 1e-10) break;
    c.swap(nxt);
  }
  return c;
}

}  // namespace

extern "C" int tq_lloyd_max(int32_t d, int32_t bits, int32_t mode, float* centroids, float* boundaries) {
  if (!centroids || !boundaries || d <= 0) return TQ_EINVAL;
  if (bits < 1 || bits > 4) return TQ_EINVAL;
  std::vector<double> c;
  if (mode == 0)
    c = lloyd_max_exact(d, bits);
  else if (mode == 1)
    c = lloyd_max_pages_trapz(d, bits);
  else
    return TQ_EINVAL;
  const int levels = 1 << bits;
  std::vector<float> c32(levels);
  for (int i = 0; i < levels; ++i) c32[i] = static_cast<float>(c[i]);
  // sort ascending (already ascending for both solvers; kept for safety)
  for (int i = 1; i < levels; ++i)
    for (int j = i; j > 0 && c32[j - 1] > c32[j]; --j) std::swap(c32[j - 1], c32[j]);
  for (int i = 0; i < levels; ++i) centroids[i] = c32[i];
  // fp32 midpoints of adjacent fp32 centroids ([API] _ensure_on_device);
  // the fp32 sum is rounded once and the halving is exact.
  for (int i = 0; i + 1 < levels; ++i) {
    volatile float s = c32[i] + c32[i + 1];
    boundaries[i] = s * 0.5f;
  }
  return TQ_OK;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): add the golden-gamma
// increment, then two xor-shift-multiply rounds and a final xor-shift.
extern "C" int tq_wht_signs(int32_t d, uint64_t seed, float* signs) {
  if (!signs || d <= 0) return TQ_EINVAL;
  uint64_t x = seed;
  for (int i = 0; i < d; ++i) {
    x += 0x9E3779B97F4A7C15ull;
    uint64_t z = x;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    signs[i] = (z >> 63) ? -1.0f : 1.0f;
  }
  return TQ_OK;
}

extern "C" int tq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                         int32_t num_kv_splits, size_t* bytes) {
  if (!bytes || batch < 0 || num_q_heads <= 0 || head_dim <= 0 || num_kv_splits <= 0) return TQ_EINVAL;
  *bytes = tq::workspace_bytes(batch, num_q_heads, head_dim, num_kv_splits);
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Argument validation (host only; shared by the launchers)
// ---------------------------------------------------------------------------

namespace tq {

size_t workspace_bytes(int64_t batch, int64_t num_q_heads, int64_t head_dim, int64_t num_kv_splits) {
  const size_t rows = static_cast<size_t>(batch) * num_q_heads * max_splits(batch, num_kv_splits);
  const size_t b = static_cast<size_t>(table_bytes(batch)) + rows * (head_dim + kPartPad) * sizeof(float);
  return (b + 255) / 256 * 256;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_store(const tq_layout* L, const void* key, const void* value, int32_t in_dtype, int64_t num_tokens,
                   int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride, const int64_t* slot_mapping,
                   const void* kv_cache, int64_t num_blocks, int32_t block_size, const float* signs,
                   const float* centroids, const float* boundaries) {
  if (!layout_consistent(L)) return L && (L->preset < 0 || L->preset >= TQ_NUM_PRESETS) ? TQ_EPRESET : TQ_EINVAL;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return TQ_EINVAL;
  if (!block_size_ok(block_size)) return TQ_EBLOCK;
  if (in_dtype != TQ_F16 && in_dtype != TQ_BF16) return TQ_EDTYPE;
  if (L->head_dim != 128 && L->head_dim != 256) return TQ_EHEADDIM;
  if (num_tokens == 0) return TQ_OK;
  if (!key || !value || !slot_mapping || !kv_cache) return TQ_EINVAL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(kv_cache) || key_tok_stride % 8 != 0 ||
      val_tok_stride % 8 != 0)
    return TQ_EINVAL;
  if (key_tok_stride < static_cast<int64_t>(num_kv_heads) * L->head_dim ||
      val_tok_stride < static_cast<int64_t>(num_kv_heads) * L->head_dim)
    return TQ_EINVAL;
  if ((!L->key_fp8 || L->value_lloyd_max) && (!signs || !centroids || !boundaries || !aligned16(signs)))
    return TQ_EINVAL;
  return TQ_OK;
}

int validate_decode(const tq_layout* L, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                    const float* signs, const float* centroids, int32_t num_kv_splits, int32_t sliding_window,
                    float value_gate, const void* workspace, size_t ws_bytes) {
  if (!layout_consistent(L)) return L && (L->preset < 0 || L->preset >= TQ_NUM_PRESETS) ? TQ_EPRESET : TQ_EINVAL;
  if (batch < 0 || num_blocks < 0 || block_table_stride < 0) return TQ_EINVAL;
  if (!block_size_ok(block_size)) return TQ_EBLOCK;
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return TQ_EGQA;
  if (q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_EDTYPE;
  if (L->head_dim != 128 && L->head_dim != 256) return TQ_EHEADDIM;
  if (num_kv_splits <= 0 || num_kv_splits > 4096 || sliding_window < 0) return TQ_EINVAL;
  if (!(value_gate >= 0.f && value_gate < 1.f)) return TQ_EINVAL;  // NaN fails too
  if (L->block_layout == TQ_LAYOUT_SOA && num_kv_heads > 8 && num_kv_heads % 8 != 0) return TQ_EUNSUPPORTED;
  if (batch == 0) return TQ_OK;
  if (!query || !kv_cache || !block_table || !seq_lens || !workspace) return TQ_EINVAL;
  if (!aligned16(query) || !aligned16(workspace) || !aligned16(kv_cache)) return TQ_EINVAL;
  if ((!L->key_fp8 || L->value_lloyd_max) && (!signs || !centroids)) return TQ_EINVAL;
  if (ws_bytes < workspace_bytes(batch, num_q_heads, L->head_dim, num_kv_splits)) return TQ_EWORKSPACE;
  return TQ_OK;
}

int validate_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                    const void* workspace, size_t ws_bytes, const void* out, int32_t out_dtype) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_splits <= 0 || num_kv_splits > 4096) return TQ_EINVAL;
  if (head_dim != 128 && head_dim != 256) return TQ_EHEADDIM;
  if (out_dtype != TQ_F16 && out_dtype != TQ_BF16 && out_dtype != TQ_F32) return TQ_EDTYPE;
  if (batch == 0) return TQ_OK;
  if (!workspace || !out || !aligned16(workspace)) return TQ_EINVAL;
  if (ws_bytes < workspace_bytes(batch, num_q_heads, head_dim, num_kv_splits)) return TQ_EWORKSPACE;
  return TQ_OK;
}

int validate_dequant(const tq_layout* L, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                     int32_t num_kv_heads, const int32_t* block_table, int32_t num_tokens, const float* signs,
                     const float* centroids, const void* key_out, const void* value_out, int32_t out_dtype,
                     int64_t out_tok_stride) {
  if (!layout_consistent(L)) return L && (L->preset < 0 || L->preset >= TQ_NUM_PRESETS) ? TQ_EPRESET : TQ_EINVAL;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return TQ_EINVAL;
  if (!block_size_ok(block_size)) return TQ_EBLOCK;
  if (out_dtype != TQ_F16 && out_dtype != TQ_BF16 && out_dtype != TQ_F32) return TQ_EDTYPE;
  if (L->head_dim != 128 && L->head_dim != 256) return TQ_EHEADDIM;
  if (num_tokens == 0) return TQ_OK;
  if (!kv_cache || !block_table || !key_out || !value_out) return TQ_EINVAL;
  if (!aligned16(kv_cache) || !aligned16(key_out) || !aligned16(value_out) || out_tok_stride % 8 != 0 ||
      out_tok_stride < static_cast<int64_t>(num_kv_heads) * L->head_dim)
    return TQ_EINVAL;
  if (static_cast<int64_t>(num_tokens) * num_kv_heads >= (int64_t{1} << 31)) return TQ_EINVAL;
  if (static_cast<int64_t>(num_tokens + block_size - 1) / block_size > num_blocks) return TQ_EINVAL;
  if ((!L->key_fp8 || L->value_lloyd_max) && (!signs || !centroids || !aligned16(signs))) return TQ_EINVAL;
  return TQ_OK;
}

}  // namespace tq

extern "C" int tq_dequant_validate(const tq_layout* layout, const void* kv_cache, int64_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads, const int32_t* block_table,
                                   int32_t num_tokens, const float* signs, const float* centroids, const void* key_out,
                                   const void* value_out, int32_t out_dtype, int64_t out_tok_stride) {
  return tq::validate_dequant(layout, kv_cache, num_blocks, block_size, num_kv_heads, block_table, num_tokens, signs,
                              centroids, key_out, value_out, out_dtype, out_tok_stride);
}

extern "C" int tq_store_validate(const tq_layout* layout, const void* key, const void* value, int32_t in_dtype,
                                 int64_t num_tokens, int32_t num_kv_heads, int64_t key_tok_stride,
                                 int64_t val_tok_stride, const int64_t* slot_mapping, const void* kv_cache,
                                 int64_t num_blocks, int32_t block_size, const float* signs, const float* centroids,
                                 const float* boundaries) {
  return tq::validate_store(layout, key, value, in_dtype, num_tokens, num_kv_heads, key_tok_stride, val_tok_stride,
                            slot_mapping, kv_cache, num_blocks, block_size, signs, centroids, boundaries);
}

extern "C" int tq_decode_validate(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache,
                                  int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                                  int32_t block_table_stride, const int32_t* seq_lens, const float* signs,
                                  const float* centroids, int32_t num_kv_splits, int32_t sliding_window,
                                  float value_gate, const void* workspace, size_t workspace_bytes, const void* out,
                                  int32_t out_dtype) {
  int st = tq::validate_decode(layout, query, q_dtype, batch, num_q_heads, num_kv_heads, kv_cache, num_blocks,
                               block_size, block_table, block_table_stride, seq_lens, signs, centroids,
                               num_kv_splits, sliding_window, value_gate, workspace, workspace_bytes);
  if (st != TQ_OK) return st;
  return tq::validate_stage2(batch, num_q_heads, layout->head_dim, num_kv_splits, workspace, workspace_bytes, out,
                             out_dtype);
}
