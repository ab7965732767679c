// Internal declarations shared by the host runtime (tq_host.cpp) and the HIP
// kernels (tq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kDim = 128;          // head_dim the kernels are specialised for
constexpr int kLutCells = 256;     // cells of the code look-up grid (see QLut)
constexpr int kMaxGroup = 4;       // q heads per kv head handled by one work-group
constexpr int kBlockTokensDev = TQ_BLOCK_TOKENS;
constexpr int kMaxPagesPerSplit = 256;   // 64 tiles of 64 tokens
constexpr int kDecodeWaves = 8;           // waves of a decode work-group (they share its tiles)
constexpr int kDecodeWgsPerCu = 1;        // decode work-groups per compute unit the split plan aims at
constexpr int kMaxPageBytes = 3200;      // largest page of any supported format (FP8 keys, 4-bit uniform values)
constexpr size_t kCounterBytes = 65536;   // arrival counters at the start of the decode workspace
// the static scratch of tq_decode_attention_noalloc: counters + 8 MiB of split partials
constexpr size_t kStaticScratchBytes = kCounterBytes + ((size_t)8 << 20);
static_assert(kStaticScratchBytes == TQ_STATIC_SCRATCH_BYTES, "tq.h states the scratch size");
// Cells of the page-append look-up grid: g = 128 y for a unit-vector coordinate
// y, cell k = round(g) + 128 in 0..256 (the end cells reach to infinity).
constexpr int kUnitCells = 257;
constexpr int kUnitCellsPadded = 260;     // a multiple of 4 (the table is copied in 16-byte units)

// One cell of the uniform grid that maps a rotated coordinate y to its code.
// The grid covers [-range, range) with kLutCells cells; `base` counts the
// thresholds lying entirely to the left of the (slightly widened) cell and `t`
// is the only threshold inside it (or +inf).  code = base + (y >= t) equals
// #{j : t_j <= y} exactly.  c_lo / c_hi are the centroids of codes base and
// base + 1, so the kernel also gets C[code] without another lookup.
struct QLut {
  int32_t base;
  float t;
  float c_lo;
  float c_hi;
};

// Constants of one context, stored in one device allocation.
struct DevConsts {
  float signs[kDim];          // +-1 of the rotation
  float kc[256];              // key centroids (fp32), 2^key_bits used
  float kt[256];              // key thresholds (fp32), 2^key_bits - 1 used (8-bit keys search them)
  float pcs1[32];             // PolarQuant: (cos, sin) of the level-1 cell centres, per code
  float pcsU[32];             // PolarQuant: (cos, sin) of the level >= 2 cell centres, per code
  float vc[16];               // value centroids (Lloyd-Max values only)
  QLut klut[kLutCells];
  QLut vlut[kLutCells];
  QLut kulut[kUnitCellsPadded];   // key grid of the page kernel; t in units of g = 128 y
  float St[kDim * kDim];      // QJL projection transposed: St[k*d + m] = S[m][k]
  // QJL projection for the page kernel's f16 MFMA: S = S_hi + S_lo (f16 terms,
  // S_lo the f16 rounding of S - S_hi).  For term t, row tile mt (rows
  // 16mt..16mt+15), K step n and lane l, the 8 halves S_t[16mt + l%16][32n +
  // 8(l/16) + e], e = 0..7, two per word (even e low), at words
  // (((t * 8 + mt) * 4 + n) * 64 + l) * 4 .. + 3.
  uint32_t Sh[2 * kDim * kDim / 2];
};

struct FieldOffsets {
  uint32_t page_bytes;
  uint32_t kcodes, knorm, ksigns, kres, vcodes, vmin, vscale;
};

struct AppendArgs {
  const void* k;
  const void* v;
  int64_t num_tokens;
  int32_t hkv;
  int32_t key_nc;             // 1: corrected norm
  const int64_t* slots;
  uint8_t* cache;
  int64_t num_blocks;
  FieldOffsets f;
  const DevConsts* c;
  uint32_t sign_bits[4];      // bit i set when sign i is -1
  float klut_scale, klut_bias;   // cell = clamp(y * scale + bias)
  float vlut_scale, vlut_bias;
  int32_t unit_grid_ok;          // kulut resolves every key threshold (the page kernel may run)
  int32_t page_wgs;              // grid of the page kernel: its resident work-groups on the device
  int32_t page_per_cu;           // resident page-kernel work-groups per compute unit
  // Round plan of the page kernel (set by its launcher): work-group w belongs to
  // slot w / slot_wgs and takes pairs in rounds r < rounds[slot]; round r's pair of
  // w is slot_wgs * sum_s min(r, rounds[s]) + w (rounds[] non-increasing).
  int32_t slot_wgs;
  int32_t rounds[3];
};

struct DecodeArgs {
  const void* q;
  int32_t q_dtype;
  const uint8_t* cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* seq_lens;
  // group: query heads per KV head (1..16); hsub = ceil(group / 4) work-groups per
  // KV head, each taking 4 consecutive query heads (the last one the rest), over
  // the same pages
  int32_t batch, max_seq, hkv, hq, group, hsub;
  int32_t xcd_pairs;          // 1: head groups of a unit on linear ids 8 apart (hsub > 1)
  float scale;                // softmax scale
  float qjl_coef;             // sqrt(pi/2) / m
  float* logits;              // may be null
  float* out;                 // [batch][hq][128]
  float* ws;                  // partials [batch][hkv * hsub][splits][4][2 + 128]
  uint32_t* counters;         // [batch][hkv * hsub] arrival counters, zero between calls
  int32_t splits;
  int32_t tiles_total;        // 64-token tiles of the longest sequence, split evenly
  FieldOffsets f;
  const DevConsts* c;
  // Fused append: the new token of sequence b ([batch][hkv][128], dtype q_dtype) is
  // position seq_lens[b] - 1; null for a plain decode.
  const void* k_new;
  const void* v_new;
  int32_t key_nc;             // 1: corrected key norm
  float klut_scale, klut_bias;
};


struct DequantArgs {
  uint32_t sign_bits[4];
  const uint8_t* cache;
  int64_t num_blocks;
  const int64_t* slots;
  const int64_t* rows;   // output row of entry i (nullptr: row i)
  int64_t n;
  int64_t buf_rows;      // rows of k_out / v_out; other rows are skipped
  int32_t hkv;
  void* k_out;           // fp32 or bf16 [buf_rows][hkv][kDim]
  void* v_out;
  FieldOffsets f;
  const DevConsts* c;
};

// Launchers (tq_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_append(const AppendArgs& a, int dtype, int key_bits, int key_mode, int val_bits,
                         int val_mode, hipStream_t s);
// Address of the decode kernel instance for a configuration (for occupancy queries).
const void* decode_kernel_ptr(int key_bits, int key_mode, int val_bits, int val_mode);
const void* append_page_kernel_ptr(int key_bits, int val_bits, bool qjl);
hipError_t launch_decode(const DecodeArgs& a, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s);
// Device address of the static decode scratch on the current device (tq_decode.hip).
hipError_t scratch_address(void** out);
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t s);
hipError_t launch_transfer(bool to_host, void* cache, void* host, const int32_t* block_ids, int64_t n,
                           int64_t num_blocks, int64_t block_bytes, int grid, hipStream_t s);
hipError_t launch_polar_keys(const AppendArgs& a, int dtype, int key_bits, hipStream_t s);
// PolarQuant keys and uniform values of few rows in one launch (one wave per row)
constexpr int64_t kPolarWaveRows = 32768;
hipError_t launch_polar_append_rows(const AppendArgs& a, int dtype, int key_bits, int val_bits, hipStream_t s);
hipError_t launch_polar_dequant(const DequantArgs& a, int key_bits, int val_bits, bool bf16_out, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, int key_bits, int key_mode, int val_bits, int val_mode, bool bf16_out,
                          hipStream_t s);

// ---- Generic path: head sizes 64 and 256 and up to 16 query heads per KV head,
// the head sizes the tuned kernels above (head_dim 128) do not take.  Same page
// format,
// same results up to the decision band and fp32 summation order (tq_generic.hip).
constexpr int kGenMaxDim = 256;
constexpr int kGenMaxGroup = 16;
constexpr int kGenMaxPageBytes = 8192;   // largest page of a generic configuration (d = 256)

struct GenConsts {
  float signs[kGenMaxDim];   // +-1 of the rotation (head_dim used)
  float kc[256];             // key centroids, 2^key_bits used
  float kt[256];             // key thresholds, 2^key_bits - 1 used, ascending
  float vc[16];              // value centroids (Lloyd-Max values)
  float vt[16];              // value thresholds (Lloyd-Max values)
};

struct GenRows {
  uint32_t kcodes, ksigns, vcodes;   // bytes per token slot of the code fields
};

struct GenAppendArgs {
  const void* k;
  const void* v;
  int32_t bf16;              // 1: bf16 inputs, 0: fp32
  int64_t num_tokens;        // rows of k / v (the batch for the one-launch step)
  int32_t hkv;
  int32_t key_bits, key_mode, val_bits, val_mode;   // key_mode: 0 plain, 1 corrected norm, 2 QJL, 3 FP8
  const int64_t* slots;      // slot of each token, or null: the new token of each sequence
  const int32_t* block_tables;   // (slots == null) new token b goes to position seq_lens[b] - 1
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t max_seq;
  uint8_t* cache;
  int64_t num_blocks;
  FieldOffsets f;
  GenRows rows;
  const GenConsts* c;
  const float* St;           // QJL: S transposed, St[k * d + m] = S[m][k]
};

struct GenDecodeArgs {
  const void* q;
  int32_t q_bf16;
  const uint8_t* cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t batch, max_seq, hkv, group;
  int32_t key_bits, key_mode, val_bits, val_mode;
  float scale;
  float qjl_coef;            // sqrt(pi/2) / d
  float* logits;             // may be null
  float* out;                // [batch][hkv * group][d]
  float* ws;                 // partials [batch][hkv][splits][group][2 + d]
  int32_t splits;
  int32_t chunk;             // tokens of one split (a multiple of 64)
  FieldOffsets f;
  GenRows rows;
  const GenConsts* c;
  const float* St;
};

struct GenDequantArgs {
  const uint8_t* cache;
  int64_t num_blocks;
  const int64_t* slots;
  const int64_t* rows;       // output row of entry i (nullptr: row i)
  int64_t n;
  int64_t buf_rows;
  int32_t hkv;
  int32_t key_bits, key_mode, val_bits, val_mode;
  void* k_out;               // fp32 or bf16 [buf_rows][hkv][d]
  void* v_out;
  int32_t bf16_out;
  FieldOffsets f;
  GenRows rows_b;
  const GenConsts* c;
};

hipError_t launch_gen_append(const GenAppendArgs& a, int d, int grid, hipStream_t s);
hipError_t launch_gen_decode(const GenDecodeArgs& a, int d, hipStream_t s);
hipError_t launch_gen_dequant(const GenDequantArgs& a, int d, int grid, hipStream_t s);

}  // namespace tq
