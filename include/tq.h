/*
 * tq.h - C ABI of the TurboQuant-style KV-cache library for MI355X (gfx950).
 *
 * What the library computes (cited by page and section; the pages are the four
 * web pages on TurboQuant KV-cache quantization):
 *   - issoh.co.jp "TurboQuantとは？vLLM・Ollama・LM Studioの対応状況と使い方",
 *     section 第1段 (stage 1): a random rotation followed by per-coordinate
 *     Lloyd-Max scalar quantization; section 第2段 (stage 2): the optional QJL
 *     1-bit residual, and the `_nc` norm correction paired with uniform value
 *     quantization; the llama.cpp section: the rotation is a normalized
 *     Walsh-Hadamard transform.
 *   - ai-navigate-news turboquant-vllm write-up, "Bugs Nobody Else Has Found":
 *     norms must be kept in fp32.
 *   - lilting.ch TurboQuant article, QJL section: sign bits of a Gaussian
 *     projection of the residual, an unbiased score correction, one projection
 *     shared by all layers and heads; the pipeline section: tokens are quantized
 *     once, online, as they arrive.
 *   - qiita article on AMD 4-bit KV caching in LMCache: two 4-bit codes per byte
 *     (element 2i in the low nibble); a reader needs the format id and version.
 *
 * Conventions for every entry point
 *   - Every call returns tq_status; nothing throws or aborts across the ABI.
 *     On failure tq_last_error_message() returns a thread-local description.
 *   - Argument errors are detected on the host, synchronously, before anything
 *     is enqueued.  Device-side work is enqueued on the caller's stream and the
 *     call returns immediately (asynchronous); faults surface at the caller's
 *     next synchronization of that stream.
 *   - The caller owns every device buffer and the stream.  The library owns only
 *     the tq_ctx (its constants live in device memory allocated by tq_create and
 *     freed by tq_destroy) and the static scratch of tq_decode_attention_noalloc.
 *     No entry point allocates device memory after tq_create.
 *   - A tq_ctx is immutable after tq_create: calls on different streams may run
 *     concurrently as long as they write disjoint memory.
 *   - Pointers marked "device" must be device-accessible (hipMalloc'd) and
 *     aligned to their element size; the cache must be 16-byte aligned.
 *
 * Cache format (TQ_FORMAT_VERSION 2)
 *   The cache is an array [num_blocks][num_kv_heads][page_bytes] of bytes.  A page
 *   holds the 16 token slots of one block for one KV head; slot = block*16 + offset.
 *   Inside a page the fields follow one another, each holding one row per slot;
 *   rows are slot-major (row of slot s at field + s*row_bytes) except the value
 *   codes (see below):
 *     key codes   d*key_bits/8 bytes per row, LSB-first bit stream (FP8 keys:
 *                 the d E4M3 bytes of the coordinates, coordinate i at byte i)
 *     key norm    fp32 (plain: ||k||; corrected: ||k|| / ||C[code]||); absent
 *                 for FP8 keys
 *     [QJL only]  sign bits d/8 bytes per row (bit i = 1 if (S r)_i >= 0), then
 *                 residual norm fp32
 *     value codes d*val_bits/8 bytes per row, LSB-first bit stream, stored
 *                 plane-major: byte p of slot s's row at field + 16*p + s
 *     uniform values: value min fp32, then value scale fp32
 *     Lloyd-Max values: value norm fp32
 *   Code i of a vector occupies stream bits [b*i, b*i+b); stream bit k is bit
 *   (k mod 8) of byte k/8.  All fp32 scalars are little-endian IEEE-754.
 *   Version history: 1 stored the value codes slot-major like the other fields;
 *   2 stores them plane-major.  A reader of transferred pages checks the version.
 *
 * Head and group sizes
 *   head_dim 128 with 1 to 16 query heads per KV head runs on the tuned kernels
 *   (the decode takes a KV head's query heads in head groups of up to 4, one
 *   work-group each, over the same pages; only the first stores the new token of
 *   a one-launch step).  head_dim 64 or 256 runs on the generic path: the same page format, entry points and results (up
 *   to the decision band and the fp32 summation order), computed by plain
 *   one-wave-per-vector append and dequantize kernels and a two-launch decode
 *   (per split, then the merge); its one-launch step is three launches (the new
 *   tokens, the decode, the merge).  The generic path takes Lloyd-Max keys (2, 3,
 *   4 or 8 bits; QJL with 2, 3 or 4), FP8 keys and both value modes; PolarQuant
 *   keys need head_dim 128 (their code
 *   order is laid out for 128 coordinates).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 1
#define TQ_FORMAT_VERSION 2
#define TQ_BLOCK_TOKENS 16

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,        /* null pointer, bad size, bad enum value      */
  TQ_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim)   */
  TQ_ERR_WORKSPACE_TOO_SMALL = 3,
  TQ_ERR_HIP = 4,                /* a HIP runtime call or launch failed         */
  TQ_ERR_OUT_OF_MEMORY = 5
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef enum {
  TQ_KEY_LLOYD = 0,      /* stage 1, stored norm = ||k||                          */
  TQ_KEY_LLOYD_NC = 1,   /* stage 1, stored norm = ||k|| / ||C[code]|| (`_nc`)     */
  TQ_KEY_LLOYD_QJL = 2,  /* stage 1 (plain norm) + 1-bit QJL residual signs        */
  TQ_KEY_FP8 = 3,        /* FP8 keys (issoh.co.jp "TurboQuantとは？…", preset table:
                            one serving preset keeps keys in FP8, values in 4 bits):
                            each coordinate of the raw key as an OCP E4M3 byte,
                            nearest value with ties to even, magnitudes above 448
                            saturate; no rotation, no per-token scalar.  Needs
                            key_bits 8 and uniform values.                        */
  TQ_KEY_POLAR = 4       /* PolarQuant keys (lilting.ch TurboQuant article,
                            PolarQuant section): after the stage-1 rotation, the
                            recursive polar transform (coordinate pairs, then pairs
                            of radii, down to one radius and d-1 angles); each
                            angle a key_bits-bit cell of a uniform grid (level 1
                            over [-pi, pi), higher levels over [0, pi/2]),
                            reconstructed at the cell centre; the radius (= ||k||)
                            in the key norm field.  Codes fill the d slots
                            subtree-major: quarter g of the coordinates owns slots
                            32g..32g+31 (its level 1..5 angles in node order; slot
                            31 holds the root, slots 63 and 95 the two level-6
                            angles, slot 127 is zero).  Uniform values only.     */
} tq_key_mode;

typedef enum {
  TQ_VAL_UNIFORM = 0,    /* per-vector fp32 min and scale, round half to even      */
  TQ_VAL_LLOYD = 1       /* same rotation + Lloyd-Max as keys, plain fp32 norm     */
} tq_val_mode;

typedef struct {
  uint32_t abi_version;   /* must equal TQ_ABI_VERSION                              */
  uint32_t head_dim;      /* d: 64, 128 or 256 (see "Head and group sizes")        */
  uint32_t num_kv_heads;  /* Hkv >= 1                                               */
  uint32_t num_q_heads;   /* Hq, a multiple of Hkv with Hq/Hkv <= 16                */
  uint32_t key_bits;      /* 2, 3 or 4 (Lloyd-Max modes); 8 (TQ_KEY_FP8)             */
  uint32_t key_mode;      /* tq_key_mode                                            */
  uint32_t val_bits;      /* 2, 3 or 4                                              */
  uint32_t val_mode;      /* tq_val_mode                                            */
  uint32_t block_tokens;  /* must equal TQ_BLOCK_TOKENS (16)                        */
} tq_config;

/* Byte layout of one page (see "Cache format").  Offsets of absent fields are
 * SIZE_MAX.  Row sizes are per token slot. */
typedef struct {
  uint32_t format_version;      /* TQ_FORMAT_VERSION                                 */
  size_t page_bytes;            /* bytes of one (block, kv head) page                */
  size_t token_head_bytes;      /* page_bytes / 16                                   */
  size_t off_kcodes, row_kcodes;
  size_t off_knorm;
  size_t off_ksigns, row_ksigns;
  size_t off_kresid;
  size_t off_vcodes, row_vcodes;
  size_t off_vmin;              /* value min (uniform) or value norm (Lloyd-Max)     */
  size_t off_vscale;            /* value scale (uniform only)                        */
} tq_layout;

typedef struct tq_ctx tq_ctx;

/* Library ABI version (TQ_ABI_VERSION of the built library). */
int tq_abi_version(void);

/* Check a configuration on the host (no GPU needed).  TQ_ERR_INVALID_ARG for
 * malformed values, TQ_ERR_UNSUPPORTED for valid ones the library does not run. */
tq_status tq_validate_config(const tq_config* cfg);

/* Page layout of a configuration, on the host (no GPU needed). */
tq_status tq_layout_for_config(const tq_config* cfg, tq_layout* out);

/* The library's own fp32 Lloyd-Max codebook for one coordinate of a rotated unit
 * vector in dimension head_dim, modelled as N(0, 1/head_dim) (issoh.co.jp page,
 * stage-1 section).  Host only.  centroids: [2^bits] ascending; thresholds:
 * [2^bits - 1] ascending midpoints (both host arrays written by the call). */
tq_status tq_codebook(uint32_t bits, uint32_t head_dim, float* centroids, float* thresholds);

/* Create a context on the current HIP device.
 *   signs_host: host [head_dim] int8, each +1 or -1 (the random signs of the
 *               rotation y = H (s * x) / sqrt(d), signs applied first).
 *   qjl_S_host: host [head_dim * head_dim] fp32 row-major (m = head_dim rows),
 *               required for TQ_KEY_LLOYD_QJL and ignored otherwise.
 * Allocates and uploads the context's device constants (synchronous).
 * On success *out owns them until tq_destroy. */
tq_status tq_create(const tq_config* cfg, const int8_t* signs_host, const float* qjl_S_host, tq_ctx** out);

/* Free a context (synchronous; the caller must not have work in flight that uses it). */
void tq_destroy(tq_ctx* ctx);

tq_status tq_layout_query(const tq_ctx* ctx, tq_layout* out);

/* Quantize num_tokens new tokens and store them in the paged cache
 * (issoh.co.jp stage-1/stage-2 sections; lilting.ch QJL and pipeline sections).
 *   k, v:         device [num_tokens][num_kv_heads][head_dim] contiguous, dtype dt
 *   slot_mapping: device int64 [num_tokens]; token t of every KV head goes to slot
 *                 slot_mapping[t] = block*16 + offset.  Slots < 0 or
 *                 >= num_blocks*16 are skipped (nothing is written for them).
 *   cache:        device [num_blocks][num_kv_heads][page_bytes]; only the rows of
 *                 the written slots change.
 * Two tokens mapped to the same slot race (the caller must not do that). */
tq_status tq_quantize_append(tq_ctx* ctx, const void* k, const void* v, tq_dtype dt, int64_t num_tokens,
                             const int64_t* slot_mapping, void* cache, int64_t num_blocks,
                             hipStream_t stream);

/* Workspace bytes tq_decode_attention needs for this batch and maximum length.
 * The first 65536 bytes of a workspace hold arrival counters that must be zero
 * before the workspace is first used (e.g. zero-fill it once when allocating);
 * every completed call leaves them zero again.  Calls that run concurrently
 * need separate workspaces. */
size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t max_seq_len);

/* Decode attention of one query token per sequence over its packed context
 * (issoh.co.jp page: the logits computed against 4-bit keys; turboquant-vllm
 * write-up: a fused attention over the compressed cache; lilting.ch QJL section:
 * the corrected score).  For q head h (kv head h / (Hq/Hkv)) and context token j:
 *   logit_j = softmax_scale * ( <q, k_hat_j>  [+ QJL correction] )
 *   out     = sum_j softmax(logit)_j * v_hat_j
 *   q:            device [batch][num_q_heads][head_dim], dtype dt
 *   cache:        as written by tq_quantize_append
 *   block_tables: device int32 [batch][max_blocks_per_seq]; token j of sequence b
 *                 is at slot block_tables[b][j/16]*16 + j%16.  Blocks outside
 *                 [0, num_blocks) are treated as empty.
 *   seq_lens:     device int32 [batch]; values are clamped to
 *                 [0, min(max_seq_len, 16*max_blocks_per_seq)].  Length 0 gives 0.
 *   out:          device fp32 [batch][num_q_heads][head_dim]
 *   logits_out:   NULL, or device fp32 [batch][num_q_heads][max_seq_len] (scaled
 *                 logits of valid tokens; other entries untouched) for testing.
 *   workspace:    device scratch of at least tq_decode_workspace_bytes bytes,
 *                 16-byte aligned, whose counter region is zero (see above);
 *                 batch * num_kv_heads must not exceed 16384 (beyond it the call
 *                 returns TQ_ERR_UNSUPPORTED before any launch). */
tq_status tq_decode_attention(tq_ctx* ctx, const void* q, tq_dtype dt, const void* cache, int64_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t batch, int32_t max_seq_len, float softmax_scale, float* out,
                              float* logits_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode attention that allocates nothing, for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  It is tq_decode_attention
 * with the split partials and arrival counters in a scratch array that the
 * library keeps in device memory (TQ_STATIC_SCRATCH_BYTES bytes per GPU, held
 * from the first tq_create on that GPU until the process ends).  Each call first
 * zeroes the counters it uses (with a kernel on `stream`), then runs the decode.
 * All calls on one GPU share that GPU's scratch, and it keeps the last call's
 * contents: calls that overlap in time on one GPU (on different streams or from
 * different threads) race and must be serialized by the caller.
 *   Arguments as for tq_decode_attention, without the workspace.
 *   Returns TQ_ERR_WORKSPACE_TOO_SMALL, before any launch, when
 *   tq_decode_workspace_bytes(ctx, batch, max_seq_len) exceeds
 *   TQ_STATIC_SCRATCH_BYTES (on the generic path, when one split's partials do
 *   not fit: it plans fewer splits to fit the scratch, which changes only the
 *   fp32 summation order); TQ_ERR_HIP when the scratch's device address could
 *   not be obtained on this GPU. */
#define TQ_STATIC_SCRATCH_BYTES (65536u + 8388608u)
tq_status tq_decode_attention_noalloc(tq_ctx* ctx, const void* q, tq_dtype dt, const void* cache, int64_t num_blocks,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                      float softmax_scale, float* out, float* logits_out, hipStream_t stream);

/* One decode step in one launch (the generic path: see "Head and group sizes"):
 * store the new token of every sequence, then
 * attend over the context including it (turboquant-vllm write-up, "Incremental
 * dequantization": each step handles only the one new token; "Bugs Nobody Else
 * Has Found": the attention is fused over the compressed cache).  The result
 * equals tq_quantize_append of the new tokens followed by tq_decode_attention,
 * up to the decision band and the fp32 summation order.
 *   k_new, v_new: device [batch][num_kv_heads][head_dim], dtype dt (the query's).
 *                 The new token of sequence b is position seq_lens[b] - 1: it is
 *                 written to slot block_tables[b][(seq_lens[b]-1)/16]*16 +
 *                 (seq_lens[b]-1)%16 (nothing is written, and the position is
 *                 attended as stored, when that block is outside [0, num_blocks);
 *                 a sequence of length 0 takes no new token).
 *   cache:        device, written at those slots only.
 *   all other arguments as for tq_decode_attention.
 * Uniform values only on the tuned path (TQ_ERR_UNSUPPORTED for Lloyd-Max values
 * there); the generic path takes both value modes. */
tq_status tq_append_decode(tq_ctx* ctx, const void* k_new, const void* v_new, const void* q, tq_dtype dt,
                           void* cache, int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float softmax_scale,
                           float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Copy whole blocks between the cache and host memory, bytes unchanged (qiita
 * LMCache article: the transfer side moves the packed slots without
 * interpreting them, and a save/restore round trip must reproduce the bytes and
 * leave other regions untouched).  A block is the num_kv_heads pages of one
 * block id: num_kv_heads * page_bytes contiguous bytes (tq_layout describes the
 * format, TQ_FORMAT_VERSION its version).
 *   block_ids: device int32 [n]; ids outside [0, num_blocks) are skipped (their
 *              host range is left as it was).
 *   host_dst / host_src: host memory pinned and mapped for the device (e.g.
 *              hipHostMalloc), 16-byte aligned, n * num_kv_heads * page_bytes
 *              bytes: block block_ids[i] <-> bytes [i * block_bytes, (i+1) *
 *              block_bytes).  The GPU reads or writes it directly over the host
 *              link; the caller synchronizes the stream before touching it.
 *   cache:     offload reads it; restore writes only the listed blocks.
 * Two ids equal in one restore race (the caller must not do that). */
tq_status tq_offload_blocks(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int32_t* block_ids, int64_t n,
                            void* host_dst, hipStream_t stream);
tq_status tq_restore_blocks(tq_ctx* ctx, const void* host_src, const int32_t* block_ids, int64_t n, void* cache,
                            int64_t num_blocks, hipStream_t stream);

/* Reconstruct stored tokens in the original basis (issoh.co.jp "TurboQuantとは？…",
 * 第1段: the rotation is orthogonal, so its inverse is diag(s) H / sqrt(d); stage 1
 * only for QJL keys):
 *   k_hat = norm * R^T C[code];  v_hat = min + scale * code  (Lloyd-Max values: as keys).
 *   slots: device int64 [n]; k_out, v_out: device fp32 [n][num_kv_heads][head_dim],
 *   16-byte aligned.  Slots outside [0, num_blocks*16) give zero rows. */
tq_status tq_dequantize(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int64_t* slots, int64_t n,
                        float* k_out, float* v_out, hipStream_t stream);

/* Incremental dequantization (turboquant-vllm write-up, "Incremental
 * dequantization": rather than reconstructing the whole cache at every step, a
 * step reconstructs only its new tokens and appends them to a running buffer):
 * entry i reconstructs the token at slots[i] into row rows[i] of k_buf / v_buf.
 *   slots:   device int64 [n]; a slot outside [0, num_blocks*16) gives a zero row.
 *   rows:    device int64 [n], or NULL for rows[i] = i.  Rows outside
 *            [0, buf_rows) are skipped; rows not listed are left as they were.
 *            Two entries naming one row race (the caller must not do that).
 *   k_buf, v_buf: device [buf_rows][num_kv_heads][head_dim] of out_dt (TQ_F32,
 *            or TQ_BF16 rounded to nearest even), 16-byte aligned; caller-owned.
 * tq_dequantize is this call with rows = NULL, buf_rows = n and TQ_F32. */
tq_status tq_dequantize_rows(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int64_t* slots, int64_t n,
                             const int64_t* rows, void* k_buf, void* v_buf, int64_t buf_rows, tq_dtype out_dt,
                             hipStream_t stream);

const char* tq_status_string(tq_status s);
const char* tq_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
