/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache store and decode attention on
 * AMD MI355X (gfx950).
 *
 * Sources (the method is defined by these pages; cited by title + section):
 *   [PR]   prhub summary of vLLM PR #38479 (TurboQuant attention backend),
 *          sections "实现拆解" (implementation breakdown) and "关键源码片段"
 *          (source excerpts: turboquant_attn.py, centroids.py,
 *          attention.py::_init_turboquant_buffers).
 *   [API]  vLLM API docs "vllm.v1.attention.backends.turboquant_attn":
 *          TurboQuantAttentionBackend, TurboQuantAttentionImpl.__init__,
 *          _ensure_on_device, do_kv_cache_update, forward, _store_kv,
 *          _continuation_prefill, _decode_attention.
 *   [TQ+]  Atlas docs "TurboQuant+ -- KV-cache compression beyond the Google
 *          baseline", sections "Background" and "What landed".
 *   [TRACK] vLLM issue #40069 "TurboQuant/HIGGS Attention follow-ups".
 *
 * Conventions shared by every entry point:
 *   - Return value: TQ_OK (0) or a negative tq_status.  Arguments are checked
 *     on the host before anything is launched; on error nothing is launched
 *     and no memory is touched.
 *   - Ownership: every pointer belongs to the caller.  "device" pointers must
 *     be GPU memory visible to the current HIP device; "host" pointers are
 *     ordinary CPU memory.  The library allocates nothing, never
 *     synchronizes the stream and never reads device memory from the host,
 *     so calls can be captured in a HIP graph (no hipMemset is issued).  Its
 *     only process-wide state is one-time set-up cached per device (the
 *     stage-1 kernels' shared-memory limit, set with hipFuncSetAttribute the
 *     first time each kernel runs on a device; the scratch address of
 *     tq_decode_attention_noalloc), kept under a lock: calls from several
 *     threads are safe, and calls that share no buffers are independent.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream).
 *     Kernels are enqueued on it; results are valid once the stream has
 *     reached them.
 *   - Element types: tq_dtype.  16-bit tensors are little-endian IEEE fp16
 *     or bfloat16.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* null pointer, negative size, misaligned tensor   */
  TQ_EPRESET = -2,      /* unknown preset id or name                        */
  TQ_EHEADDIM = -3,     /* head_dim unsupported (kernels: 128, 256)         */
  TQ_EBLOCK = -4,       /* block_size not one of 16, 32, 64, 128            */
  TQ_EGQA = -5,         /* num_q_heads not a multiple of num_kv_heads       */
  TQ_EWORKSPACE = -6,   /* workspace smaller than tq_decode_workspace_bytes */
  TQ_EDTYPE = -7,       /* element type not allowed for that argument       */
  TQ_EHIP = -8,         /* a HIP launch failed (hipGetLastError)            */
  TQ_EUNSUPPORTED = -9  /* valid but unsupported combination                */
} tq_status;

/* Presets: [PR] "实现拆解" item 1; [API] TurboQuantAttentionBackend
 * supported_kv_cache_dtypes.  k8v4 = FP8 (E4M3) keys + 4-bit values;
 * 4bit_nc = 4-bit Lloyd-Max keys + 4-bit values; k3v4_nc = 3-bit keys +
 * 4-bit values; 3bit_nc = 3-bit keys + 3-bit values; "nc" = norm
 * correction (stored key norm is ||x|| / ||c[code]||, [TQ+] "Background").
 * More codecs ([TQ+] "What landed": the 2-bit Lloyd-Max codebook, 4 codes
 * per byte, and asymmetric K/V pairs): k8v3 = FP8 keys + 3-bit values;
 * k4v3_nc = 4-bit keys + 3-bit values; 2bit_nc = 2-bit keys + 2-bit values.
 * Names "turboquant_k8v3", "turboquant_k4v3_nc", "turboquant_2bit_nc".
 * Lloyd-Max values ([TQ+] "What landed": values take the keys' rotation and
 * Lloyd-Max codebook with the matched-norm correction): k8v3lm = FP8 keys +
 * 3-bit Lloyd-Max values; 3bit_lm = 3-bit keys + 3-bit Lloyd-Max values;
 * at the other widths of the pages' turbo2/3/4 family: k8v4lm = FP8 keys +
 * 4-bit Lloyd-Max values; 4bit_lm = 4-bit keys + 4-bit Lloyd-Max values;
 * 2bit_lm = 2-bit keys + 2-bit Lloyd-Max values.  Names
 * "turboquant_k8v3lm", "turboquant_3bit_lm", "turboquant_k8v4lm",
 * "turboquant_4bit_lm", "turboquant_2bit_lm". */
typedef enum {
  TQ_K8V4 = 0,
  TQ_4BIT_NC = 1,
  TQ_K3V4_NC = 2,
  TQ_3BIT_NC = 3,
  TQ_K8V3 = 4,
  TQ_K4V3_NC = 5,
  TQ_2BIT_NC = 6,
  TQ_K8V3LM = 7,
  TQ_3BIT_LM = 8,
  TQ_K8V4LM = 9,
  TQ_4BIT_LM = 10,
  TQ_2BIT_LM = 11,
  TQ_NUM_PRESETS = 12
} tq_preset;

typedef enum { TQ_F16 = 0, TQ_BF16 = 1, TQ_F32 = 2 } tq_dtype;

/* Byte layout of one combined slot (one token, one KV head):
 *   MSE keys: [key codes (key_data_bytes) | fp16 key norm] [value codes
 *             (value_data_bytes) | fp16 scale | fp16 zero] [pad to even]
 *   FP8 keys: [head_dim x fp8 key] [value region] [pad]
 * key_data_bytes = ceil(head_dim*key_bits/8) (head_dim for FP8),
 * value_data_bytes = ceil(head_dim*value_bits/8), slot_size_aligned =
 * slot_size rounded up to even ([API] TurboQuantAttentionImpl.__init__ and
 * _continuation_prefill; [PR] get_kv_cache_shape).  Codes are packed as one
 * little-endian bit stream, code j in bits [b*j, b*j+b) (3-bit: 8 codes per
 * 3 bytes, [TQ+] "Background"). */
/* Block byte conventions of the cache; both give the same tensor shape.
 *   TQ_LAYOUT_AOS: the combined slots above, slot m of KV head h at byte
 *     (m*num_kv_heads + h)*slot_size_aligned.
 *   TQ_LAYOUT_SOA: per cache block of block_size tokens, a data region of
 *     block_size*num_kv_heads rows (row r = t*num_kv_heads + h, token t of
 *     the block) of soa_data_bytes = key_data_bytes + value_data_bytes each,
 *     [key data | value codes]; then, at byte block_size*num_kv_heads*
 *     soa_data_bytes of the block, soa_meta_fields little-endian 16-bit
 *     fields per row, field f of row r at 2*(r*soa_meta_fields + f): MSE keys
 *     (norm, scale, zero), FP8 keys (scale, zero).  ([API] _store_kv: data
 *     and metadata regions separated per block, same tensor shape; forward:
 *     such a cache must be read by the matching reader; _continuation_prefill:
 *     data bytes per slot, metadata region offset, field counts and indices.
 *     Row order and field interleave are this library's reading: the pages
 *     give only those constants.)
 * A cache is written and read with one convention: every call takes it from
 * the layout, so the store, decode and dequant of one layout agree. */
typedef enum { TQ_LAYOUT_AOS = 0, TQ_LAYOUT_SOA = 1 } tq_block_layout;

typedef struct tq_layout {
  int32_t preset;
  int32_t head_dim;
  int32_t key_fp8;
  int32_t key_bits;        /* 8 for FP8 keys */
  int32_t value_bits;
  int32_t norm_correction;
  int32_t n_centroids;     /* 2^key_bits, 0 for FP8 keys */
  int32_t key_data_bytes;
  int32_t key_packed_size;
  int32_t value_data_bytes;
  int32_t value_packed_size;
  int32_t slot_size;
  int32_t slot_size_aligned;
  int32_t block_layout;    /* tq_block_layout */
  int32_t soa_data_bytes;  /* SoA: key_data_bytes + value_data_bytes; 0 for AoS */
  int32_t soa_meta_fields; /* SoA: 3 (MSE keys) or 2 (FP8 keys); one fewer with Lloyd-Max values; 0 for AoS */
  int32_t value_lloyd_max; /* 1: values are rotated Lloyd-Max codes + fp16 norm (value region [codes |
                              norm]); 0: uniform codes + fp16 scale + fp16 zero */
} tq_layout;

/* Library version string (static storage). */
const char* tq_version(void);

/* Human-readable text for a tq_status (static storage). */
const char* tq_status_str(int status);

/* Text of the HIP error behind the most recent TQ_EHIP returned on this
 * thread ("no error" if there was none); static storage. */
const char* tq_last_hip_error(void);

/* "turboquant_k8v4" | "turboquant_4bit_nc" | "turboquant_k3v4_nc" |
 * "turboquant_3bit_nc" | "turboquant_k8v3" | "turboquant_k4v3_nc" |
 * "turboquant_2bit_nc" | "turboquant_k8v3lm" | "turboquant_3bit_lm" ->
 * preset id (host).  TQ_EPRESET for other names. */
int tq_preset_from_name(const char* name, int32_t* preset);

/* Fill *out for (preset, head_dim) (host), block_layout TQ_LAYOUT_AOS.
 * head_dim must be a positive multiple of 8; the kernels additionally need
 * head_dim 128 or 256.  A 256-dim slot keeps the same field order: its key
 * bits and value codes are positional (dim i at bits B*i), so their first
 * half is what a 128-dim slot of the first 128 dims would hold; the rotation
 * is the 256-point transform and the codebook the one for d = 256 (the
 * marginal N(0, 1/d) of tq_lloyd_max; [TQ+] "What landed" ships sign arrays
 * for 256-dim heads). */
int tq_layout_init(int32_t preset, int32_t head_dim, tq_layout* out);

/* tq_layout_init with a block convention (tq_block_layout) (host).  TQ_EINVAL
 * for an unknown convention.  Decode attention over an SoA cache needs
 * num_kv_heads <= 8 or a multiple of 8 (TQ_EUNSUPPORTED otherwise); store
 * and dequant take any head count. */
int tq_layout_init_ex(int32_t preset, int32_t head_dim, int32_t block_layout, tq_layout* out);

/* Cache tensor shape (num_blocks, block_size, num_kv_heads,
 * slot_size_aligned), no leading K/V dimension ([PR] get_kv_cache_shape),
 * for either block convention.  The cache is a byte tensor of that shape
 * (host). */
int tq_kv_cache_shape(const tq_layout* layout, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int64_t shape_out[4]);

/* Lloyd-Max codebook for the rotated-coordinate marginal N(0, 1/d) ([PR]
 * "关键源码片段", centroids.py), host.  mode 0 = exact (closed-form Gaussian
 * cell means iterated to a float64 fixed point, antisymmetric); mode 1 =
 * the pages' trapezoid solver (200 intervals, cells closed at +-10.5 sigma,
 * 200 rounds, tol 1e-10).  Writes 2^bits fp32 centroids (ascending) and
 * 2^bits - 1 fp32 boundaries = fp32 midpoints of adjacent fp32 centroids
 * ([API] _ensure_on_device).  bits in 1..4. */
int tq_lloyd_max(int32_t d, int32_t bits, int32_t mode, float* centroids, float* boundaries);

/* d Rademacher signs (+1.0f / -1.0f) for the rotation (host): sign i is -1
 * when the top bit of the i-th SplitMix64 output from `seed` is set.  The
 * pages derive a per-layer seed ([PR] attention.py excerpt); the caller owns
 * that policy. */
int tq_wht_signs(int32_t d, uint64_t seed, float* signs);

/* Bytes of device workspace tq_decode_attention needs ([PR] attention.py
 * excerpt, the mid_o buffer of stage-1 partials; [API] _decode_attention).
 * Layout (library-private; callers treat it as scratch):
 *   int32 [batch][2] table = (first work unit, number of work units) of each
 *   sequence, padded to 256 bytes; then fp32 rows [U][num_q_heads][head_dim
 *   + 4] = the normalized partial output of (unit, query head), its
 *   natural-log LSE and 3 pad floats.  U = batch * S_max, S_max =
 *   num_kv_splits * max(1, ceil(512 / (batch * num_kv_splits))).
 * At least the pages' (batch, num_q_heads, num_kv_splits, head_dim + 1)
 * fp32 buffer.  Rounded up to 256.  One workspace can serve every layer
 * (calls on one stream run in order). */
int tq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                              size_t* bytes);

/* Quantize num_tokens new K/V rows and write their slots ([API]
 * do_kv_cache_update / _store_kv; [PR] "实现拆解" item 4: one fused launch).
 * Per (token n, KV head h):
 *   MSE keys: nu = ||k||, y = H (s .* k) / sqrt(D) (s = signs, H the
 *     Sylvester Walsh-Hadamard matrix), code_i = #{j : boundaries[j] < y_i/nu},
 *     stored norm = nu / ||centroids[code]|| (norm correction) or nu;
 *   FP8 keys: E4M3 round-to-nearest-even, saturating at +-448;
 *   values: zero = fp16(min v), scale = fp16((max v - min v)/(2^b - 1)),
 *     code = clamp(floor(fl32(fl32(v - zero) * fl32(1/scale)) + 0.5)).
 * Arguments:
 *   key, value       device, dtype in_dtype (TQ_F16 | TQ_BF16); row (n, h)
 *                    starts at element n*key_tok_stride + h*head_dim (heads
 *                    contiguous); base 16-byte aligned, strides multiples of 8.
 *   num_tokens       N >= 0; N == 0 returns TQ_OK with no launch.
 *   slot_mapping     device int64 [N]; slot m < 0 skips the token.
 *   kv_cache         device bytes, shape tq_kv_cache_shape(...).  Only the
 *                    addressed slots are written.  Slots must be distinct
 *                    (two tokens mapped to one slot race).
 *   signs            device fp32 [head_dim] (MSE keys or Lloyd-Max values;
 *                    may be NULL otherwise).
 *   centroids        device fp32 [n_centroids]; boundaries device fp32
 *                    [n_centroids - 1] (MSE presets; NULL for FP8 keys).
 *                    Lloyd-Max value layouts append the value codebook:
 *                    centroids [key codebook (MSE keys) | 2^value_bits],
 *                    boundaries [key boundaries | 2^value_bits - 1]; the
 *                    decode and dequant read centroids the same way.
 * Supported: head_dim 128 or 256, block_size 16/32/64/128, num_kv_heads >= 1. */
int tq_store(const tq_layout* layout, const void* key, const void* value, int32_t in_dtype, int64_t num_tokens,
             int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride, const int64_t* slot_mapping,
             void* kv_cache, int64_t num_blocks, int32_t block_size, const float* signs, const float* centroids,
             const float* boundaries, void* stream);

/* Host-only check of tq_store's arguments (no launch, no device access). */
int tq_store_validate(const tq_layout* layout, const void* key, const void* value, int32_t in_dtype,
                      int64_t num_tokens, int32_t num_kv_heads, int64_t key_tok_stride, int64_t val_tok_stride,
                      const int64_t* slot_mapping, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                      const float* signs, const float* centroids, const float* boundaries);

/* Decode attention of one query per sequence over the compressed cache
 * ([API] _decode_attention; [PR] "实现拆解" item 4: stage 1 scores and
 * accumulates values per KV split, stage 2 merges the splits with a
 * log-sum-exp reduction).  Query head hq reads KV head hq / (Hq/Hk).  MSE
 * keys are scored against the query rotated by the same transform;
 * FP8 keys against the raw query.  Result = softmax(scale * q.k) v over
 * tokens [w_b, seq_lens[b]) of each sequence, w_b the window start; an empty
 * range gives o = 0 and lse = -inf (lse = the sink with sinks).
 * Arguments:
 *   query        device [batch, num_q_heads, head_dim], dtype q_dtype
 *                (TQ_F16 | TQ_BF16), contiguous.
 *   kv_cache     device bytes written by tq_store (same layout, block_size).
 *   block_table  device int32 [batch, block_table_stride]; entries past
 *                ceil(seq_lens[b]/block_size) are never read.
 *   seq_lens     device int32 [batch], each in [0, block_table_stride*block_size].
 *   signs, centroids  as for tq_store (MSE presets).
 *   scale        softmax scale (1/sqrt(head_dim) for standard attention).
 *   num_kv_splits S >= 1: the split-KV parallelism requested.  The library
 *                launches batch * S_int work units (S <= S_int <= S_max,
 *                raised so the grid has about 512 workgroups, capped by
 *                block_table_stride) and gives each sequence a number of
 *                units in proportion to its length, each a contiguous range
 *                of 16-token tiles; the launch shape depends only on the
 *                arguments, never on device data.
 *   sliding_window  > 0: each query sees the last sliding_window tokens of
 *                its sequence, itself included (w_b = max(0, seq_len -
 *                sliding_window)); 0: the whole sequence.  ([API]
 *                TurboQuantAttentionImpl.__init__ keeps sliding_window and
 *                _decode_attention hands it to the decode kernel; the window
 *                reading is this library's.)  Tiles before the window are
 *                neither read nor counted in the work split.
 *   value_gate   0: exact attention.  In (0, 1): the opt-in sparse-V gate
 *                ([TQ+] "nvfp4 dec_after_8K cliff explained": rows whose
 *                softmax factor exp(s - m) falls below the gate contribute
 *                no value; 1e-3 there).  A token whose factor against the
 *                exact running maximum of its query head (over the tokens
 *                its work unit has scored so far) is below value_gate keeps
 *                its weight in the softmax denominator (and the lse) but
 *                adds no value; a pair of 16-token tiles whose tokens are all
 *                gated skips its value decode and value products.  The
 *                running maximum never exceeds the final one, so every gated
 *                token has exp(s - max) < value_gate and the output moves by
 *                at most sum over such tokens of (normalized weight) * |v|.
 *                The cache bytes are read either way (tiles arrive whole),
 *                so the gate saves no memory traffic; on the workloads
 *                measured here it costs time rather than saving it.
 *                TQ_EINVAL outside [0, 1) or NaN.
 *   sinks        device fp32 [num_q_heads] attention-sink logits, or NULL
 *                ([API] TurboQuantAttentionImpl.__init__ / _decode_attention
 *                pass per-head sinks).  Reading: one more logit in each
 *                head's softmax denominator, in the units of scale * q.k,
 *                with no value: o = sum_t e^{s_t} v_t / (sum_t e^{s_t} +
 *                e^{sink}); the lse includes it.  Applied in stage 2.
 *   workspace    device, >= tq_decode_workspace_bytes(batch, num_q_heads,
 *                head_dim, S) bytes, 16-byte aligned; contents are scratch.
 *   out          device [batch, num_q_heads, head_dim], dtype out_dtype
 *                (TQ_F16 | TQ_BF16 | TQ_F32), contiguous.
 *   lse_out      device fp32 [batch, num_q_heads] natural-log LSE, or NULL.
 * Supported: head_dim 128 or 256, block_size 16/32/64/128, num_q_heads a
 * multiple of num_kv_heads, sliding_window >= 0, 0 <= value_gate < 1
 * (TQ_EINVAL otherwise). */
int tq_decode_attention(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks,
                        int32_t block_size, const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* seq_lens, const float* signs, const float* centroids, float scale,
                        int32_t num_kv_splits, int32_t sliding_window, float value_gate, const float* sinks,
                        void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype, float* lse_out,
                        void* stream);

/* Host-only check of tq_decode_attention's arguments. */
int tq_decode_validate(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks,
                       int32_t block_size, const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, const float* signs, const float* centroids, int32_t num_kv_splits,
                       int32_t sliding_window, float value_gate, const void* workspace, size_t workspace_bytes,
                       const void* out, int32_t out_dtype);

/* The two launches of tq_decode_attention, exposed separately so that each
 * can be timed on its own.  Stage 1 writes the workspace table and the
 * partial rows of every work unit; stage 2 merges each sequence's units into
 * out / lse_out.  Same arguments and checks as tq_decode_attention (stage 1
 * takes the window and the value gate, stage 2 the sinks); stage 2 must run
 * on a workspace written by stage 1 with the same batch, num_q_heads and
 * head_dim. */
int tq_decode_stage1(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                     const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                     const float* signs, const float* centroids, float scale, int32_t num_kv_splits,
                     int32_t sliding_window, float value_gate, void* workspace, size_t workspace_bytes,
                     void* stream);

int tq_decode_stage2(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_kv_splits,
                     const float* sinks, const void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                     float* lse_out, void* stream);

/* Decode attention that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It makes the same
 * two launches as tq_decode_attention, with the same results, but the stage-1
 * sequence table and partial rows live in a scratch array that libtq holds
 * in device memory for the life of the process: TQ_NOALLOC_SCRATCH_BYTES on
 * each device the library runs on (a file-scope device array; its address
 * is looked up once per device, on the first call with that device current,
 * and cached).  Arguments: as for tq_decode_attention without workspace and
 * workspace_bytes.  Errors: as for tq_decode_attention, and TQ_EWORKSPACE
 * (nothing launched) when tq_decode_workspace_bytes(batch, num_q_heads,
 * head_dim, num_kv_splits) exceeds TQ_NOALLOC_SCRATCH_BYTES; TQ_EHIP if the
 * scratch address cannot be obtained.  Nothing in the scratch needs to start
 * at zero (stage 1 writes every entry stage 2 reads).  Every call on a GPU
 * shares that GPU's scratch and leaves the last call's contents in it: calls
 * that overlap on one GPU (different streams or threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * No hipMalloc, hipFree or allocating library routine is called. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int tq_decode_attention_noalloc(const tq_layout* layout, const void* query, int32_t q_dtype, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads, const void* kv_cache, int64_t num_blocks,
                                int32_t block_size, const int32_t* block_table, int32_t block_table_stride,
                                const int32_t* seq_lens, const float* signs, const float* centroids, float scale,
                                int32_t num_kv_splits, int32_t sliding_window, float value_gate, const float* sinks,
                                void* out, int32_t out_dtype, float* lse_out, void* stream);

/* Dequantize the cached prefix of one sequence back to dense K and V in the
 * original space, the first step of a continuation prefill ([API]
 * _continuation_prefill: the cached K/V are dequantized, MSE keys rotated
 * back, then attention runs over cached + new tokens).  For tokens
 * t < num_tokens (token t in block block_table[t / block_size] at offset
 * t % block_size) and KV heads h:
 *   MSE keys: k = s .* (H (gamma c[code])) / sqrt(D), the transpose of the
 *             store's rotation applied to the dequantized rotated key;
 *   FP8 keys: the E4M3 values;
 *   values:   zero + scale * code (stored fp16 scale and zero).
 * Computed in fp32 and rounded to nearest even in out_dtype.
 * Arguments:
 *   kv_cache      device bytes written by tq_store (same layout, block_size).
 *   block_table   device int32 [ceil(num_tokens / block_size)], entries < num_blocks.
 *   num_tokens    >= 0; 0 returns TQ_OK with no launch.
 *   signs, centroids  as for tq_store (MSE presets; may be NULL for FP8 keys).
 *   key_out, value_out  device, row (t, h) at element t*out_tok_stride + h*head_dim,
 *                 dtype out_dtype (TQ_F16 | TQ_BF16 | TQ_F32), 16-byte aligned;
 *                 out_tok_stride >= num_kv_heads * head_dim and a multiple of 8,
 *                 so the rows can land in a larger [tokens, Hk, D] buffer.  Only
 *                 the rows written are touched.
 * Supported: head_dim 128 or 256, block_size 16/32/64/128, num_tokens * num_kv_heads < 2^31. */
int tq_dequant_kv(const tq_layout* layout, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, const int32_t* block_table, int32_t num_tokens, const float* signs,
                  const float* centroids, void* key_out, void* value_out, int32_t out_dtype, int64_t out_tok_stride,
                  void* stream);

/* Host-only check of tq_dequant_kv's arguments. */
int tq_dequant_validate(const tq_layout* layout, const void* kv_cache, int64_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, const int32_t* block_table, int32_t num_tokens, const float* signs,
                        const float* centroids, const void* key_out, const void* value_out, int32_t out_dtype,
                        int64_t out_tok_stride);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
