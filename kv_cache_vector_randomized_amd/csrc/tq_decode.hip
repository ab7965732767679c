// Decode attention over the packed cache for gfx950 (one launch, split merge included).
//
// Sources (page and section): issoh.co.jp "TurboQuantとは？…", the section on
// where the zero-loss claim comes from (logits against 4-bit keys are the part
// that is sped up); ai-navigate-news turboquant-vllm write-up (attention has to
// be fused over the compressed cache); lilting.ch TurboQuant article, QJL section
// (query kept in full precision, projected with the same S; corrected score).
//
// One work-group per (split of the context, kv head, sequence); each wave owns
// 64-token tiles (4 pages).  Lane l holds token l's packed key row (prefetched one
// tile ahead); codes become centroids through a 16-entry LDS table and are
// contracted with the group's 4 rotated query heads on the fp32 4x4x1 (16-block)
// MFMA, which keeps exact fp32 products.  Value codes are stored plane-major in a
// page (byte p of the 16 slots is contiguous), so lane l loads the byte plane of
// its two coordinates for 16 tokens with one coalesced 16-byte load per page and
// converts four tokens per 32-bit word.  The online softmax runs per lane; the
// weights are contracted with the value codes on the same MFMA.  Per-split
// partials (max, sum, 128 outputs) go to the workspace; the last work-group of
// each (sequence, kv head) to finish, found with a self-resetting arrival
// counter, merges them by log-sum-exp and writes the output.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide max: DPP within rows of 16 lanes, then the four row results.
// Rows outside ROW_MASK keep their own value, which is neutral for max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<0xB1, 0xF>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E, 0xF>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141, 0xF>(v));   // row_half_mirror
  v = fmaxf(v, dpp<0x140, 0xF>(v));   // row_mirror: every lane of a row holds the row max
  v = fmaxf(v, dpp<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
  v = fmaxf(v, dpp<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3: lane 63 holds the max
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Value codes of coordinates 2*lane, 2*lane+1 for the four tokens of one 32-bit
// word of the lane's byte plane(s): returns (lo, hi) with one code per byte.
template <int VB>
__device__ __forceinline__ void value_nibbles(uint32_t x0, uint32_t x1, int sh, uint32_t& lo, uint32_t& hi) {
  if constexpr (VB == 4) {
    lo = x0 & 0x0F0F0F0Fu;
    hi = (x0 >> 4) & 0x0F0F0F0Fu;
  } else if constexpr (VB == 2) {
    const uint32_t f = (x0 >> sh) & 0x0F0F0F0Fu;
    lo = f & 0x03030303u;
    hi = (f >> 2) & 0x03030303u;
  } else {
    // 6-bit field per byte: bits [sh, 8) of plane p0 and [0, sh - 2) of plane p0 + 1
    const uint32_t m1 = (0xFFu >> sh) * 0x01010101u;
    const uint32_t m2 = ((0xFFu << (8 - sh)) & 0xFFu) * 0x01010101u;
    const uint32_t f = (((x0 >> sh) & m1) | ((x1 << (8 - sh)) & m2)) & 0x3F3F3F3Fu;
    lo = f & 0x07070707u;
    hi = (f >> 3) & 0x07070707u;
  }
}

template <int KB, int VB>
struct TileRegs {
  uint32_t kw[KB * 4];          // this lane's key row
  float knorm, va, vb, kres;
  uint4 sg;
};

// Block ids of the 4 pages of one tile (wave-uniform; -1: absent or out of range).
struct TilePages {
  int b[4];
};

// The wave keeps the block ids of all its tiles in one register: lane 4k + pg
// holds page pg of the wave's k-th tile.  lane_block returns the block id of the
// page that lane `lane` reads in the k-th tile (lanes 16*pg .. 16*pg+15 read page
// pg), fetched across lanes without a branch.
__device__ __forceinline__ int lane_block(int blk_reg, int k, int lane) {
  return __builtin_amdgcn_ds_bpermute((4 * k + (lane >> 4)) << 2, blk_reg);
}

__device__ __forceinline__ TilePages pages_of(int blk_reg, int k) {
  TilePages p;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) p.b[pg] = __builtin_amdgcn_readlane(blk_reg, 4 * k + pg);
  return p;
}

// Loads of one 64-token tile (4 pages of one kv head).  Loads are unconditional:
// an absent page (block id -1) reads block 0 in its place and the lanes of
// absent pages and of tokens past the end are masked after the loads, which
// keeps the load path free of branches.  The caller guarantees num_blocks >= 1.
__device__ __forceinline__ int64_t page_offset(int blk, int kvh, int64_t blk_stride, int64_t head_stride) {
  return (int64_t)(blk >= 0 ? blk : 0) * blk_stride + kvh * head_stride;
}

template <int KB, bool QJL, int VB, bool VLM>
__device__ __forceinline__ void load_tile(TileRegs<KB, VB>& r, const DecodeArgs& a, int blk, int kvh, int lane,
                                          int64_t blk_stride, int64_t head_stride) {
  constexpr int KROW = kDim * KB / 8;
  const uint8_t* page = a.cache + page_offset(blk, kvh, blk_stride, head_stride);
  const int so = lane & 15;
  const uint4* src = reinterpret_cast<const uint4*>(page + a.f.kcodes + so * KROW);
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    const uint4 u = src[j];
    r.kw[4 * j] = u.x; r.kw[4 * j + 1] = u.y; r.kw[4 * j + 2] = u.z; r.kw[4 * j + 3] = u.w;
  }
  r.knorm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
  r.va = reinterpret_cast<const float*>(page + a.f.vmin)[so];
  r.vb = VLM ? 0.f : reinterpret_cast<const float*>(page + a.f.vscale)[so];
  if (QJL) {
    r.sg = reinterpret_cast<const uint4*>(page + a.f.ksigns)[so];
    r.kres = reinterpret_cast<const float*>(page + a.f.kres)[so];
  } else {
    r.sg = make_uint4(0u, 0u, 0u, 0u);
    r.kres = 0.f;
  }
}

// Lloyd-Max values: byte plane(s) of this lane's two coordinates for the tile's
// 4 pages (16 tokens per page, one coalesced 16-byte load per page and plane).
template <int VB>
__device__ __forceinline__ void load_value_planes(uint4 (&vp)[VB == 3 ? 8 : 4], const DecodeArgs& a,
                                                  const TilePages& tp, int kvh, int lane, int64_t blk_stride,
                                                  int64_t head_stride) {
  constexpr int VROW = kDim * VB / 8;
  const int p0 = (VB == 4) ? lane : (VB == 2) ? (lane >> 1) : ((6 * lane) >> 3);
  const int p1 = (6 * lane >> 3) + 1 < VROW ? (6 * lane >> 3) + 1 : VROW - 1;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {
    const uint8_t* vbase = a.cache + page_offset(tp.b[pg], kvh, blk_stride, head_stride) + a.f.vcodes;
    vp[pg] = *reinterpret_cast<const uint4*>(vbase + p0 * 16);
    if constexpr (VB == 3) vp[4 + pg] = *reinterpret_cast<const uint4*>(vbase + p1 * 16);
  }
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Uniform values: lane l loads, from page l/16 of the tile, the byte planes of
// coordinates 8j..8j+7 (j = l%16): VB planes of 16 slots, contiguous in the page.
template <int VB>
__device__ __forceinline__ void load_value_group(uint4 (&vq)[VB], const DecodeArgs& a, int blk, int kvh, int lane,
                                                 int64_t blk_stride, int64_t head_stride) {
  const uint4* src = reinterpret_cast<const uint4*>(a.cache + page_offset(blk, kvh, blk_stride, head_stride) +
                                                    a.f.vcodes + 16 * VB * (lane & 15));
#pragma unroll
  for (int i = 0; i < VB; ++i) vq[i] = src[i];
}

typedef int intx4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


// Wave-wide maxima of five values at once.  Each DPP step combines a lane with
// another lane of its row (quad swaps, half-row and row mirrors), then the row
// broadcasts carry row 0 into row 1, row 2 into row 3 and rows 0-1 into rows
// 2-3, so lane 63 ends with the maximum.  The five reductions are interleaved,
// so every DPP source was written at least four instructions earlier (the DPP
// read-after-write hazard needs two); the leading s_nop covers the producers.
__device__ __forceinline__ void wave_max5(float& v0, float& v1, float& v2, float& v3, float& v4) {
#define TQ_DPP5(CTL)                                                   \
  "v_max_f32_dpp %0, %0, %0 " CTL "\n\t"                               \
  "v_max_f32_dpp %1, %1, %1 " CTL "\n\t"                               \
  "v_max_f32_dpp %2, %2, %2 " CTL "\n\t"                               \
  "v_max_f32_dpp %3, %3, %3 " CTL "\n\t"                               \
  "v_max_f32_dpp %4, %4, %4 " CTL "\n\t"
  asm volatile("s_nop 1\n\t"
               TQ_DPP5("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf")
               TQ_DPP5("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf")
               TQ_DPP5("row_half_mirror row_mask:0xf bank_mask:0xf")
               TQ_DPP5("row_mirror row_mask:0xf bank_mask:0xf")
               TQ_DPP5("row_bcast:15 row_mask:0xa bank_mask:0xf")
               TQ_DPP5("row_bcast:31 row_mask:0xc bank_mask:0xf")
               "s_nop 1"
               : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3), "+v"(v4));
#undef TQ_DPP5
  v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v0), 63));
  v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v1), 63));
  v2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v2), 63));
  v3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v3), 63));
  v4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v4), 63));
}

// Wave-wide sums of eight values at once, with the same DPP pattern as
// wave_max5 (a lane is always combined with a lane of the complementary group,
// so nothing is counted twice); lane 63 ends with the totals.
__device__ __forceinline__ void wave_sum8(float (&v)[8]) {
#define TQ_DPP8(CTL)                                                   \
  "v_add_f32_dpp %0, %0, %0 " CTL "\n\t"                               \
  "v_add_f32_dpp %1, %1, %1 " CTL "\n\t"                               \
  "v_add_f32_dpp %2, %2, %2 " CTL "\n\t"                               \
  "v_add_f32_dpp %3, %3, %3 " CTL "\n\t"                               \
  "v_add_f32_dpp %4, %4, %4 " CTL "\n\t"                               \
  "v_add_f32_dpp %5, %5, %5 " CTL "\n\t"                               \
  "v_add_f32_dpp %6, %6, %6 " CTL "\n\t"                               \
  "v_add_f32_dpp %7, %7, %7 " CTL "\n\t"
  asm volatile("s_nop 1\n\t"
               TQ_DPP8("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf")
               TQ_DPP8("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf")
               TQ_DPP8("row_half_mirror row_mask:0xf bank_mask:0xf")
               TQ_DPP8("row_mirror row_mask:0xf bank_mask:0xf")
               TQ_DPP8("row_bcast:15 row_mask:0xa bank_mask:0xf")
               TQ_DPP8("row_bcast:31 row_mask:0xc bank_mask:0xf")
               "s_nop 1"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#undef TQ_DPP8
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// Value codes of this lane's page and coordinates 8j..8j+7 (j = lane % 16) as
// the B operand of the int8 MFMA for coordinate 8j + m: one code per byte, byte s
// of dword w is slot 4w + s of the page.  Codes are packed LSB-first, so within a
// byte plane the shifts and masks below act on four slots at once.
template <int VB, int M>
__device__ __forceinline__ intx4 value_codes(const uint4 (&vq)[VB]) {
  uint32_t r[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (VB == 4) {
      const uint32_t x = u4get(vq[M >> 1], w);
      r[w] = (M & 1) ? ((x >> 4) & 0x0F0F0F0Fu) : (x & 0x0F0F0F0Fu);
    } else if constexpr (VB == 2) {
      const uint32_t x = u4get(vq[M >> 2], w);
      r[w] = (x >> (2 * (M & 3))) & 0x03030303u;
    } else {
      // 8 codes of 3 bits span the three planes p0, p1, p2 of the group
      const uint32_t p0 = u4get(vq[0], w), p1 = u4get(vq[1], w), p2 = u4get(vq[2], w);
      if constexpr (M == 0) r[w] = p0 & 0x07070707u;
      else if constexpr (M == 1) r[w] = (p0 >> 3) & 0x07070707u;
      else if constexpr (M == 2) r[w] = ((p0 >> 6) & 0x03030303u) | ((p1 << 2) & 0x04040404u);
      else if constexpr (M == 3) r[w] = (p1 >> 1) & 0x07070707u;
      else if constexpr (M == 4) r[w] = (p1 >> 4) & 0x07070707u;
      else if constexpr (M == 5) r[w] = ((p1 >> 7) & 0x01010101u) | ((p2 << 1) & 0x06060606u);
      else if constexpr (M == 6) r[w] = (p2 >> 2) & 0x07070707u;
      else r[w] = (p2 >> 5) & 0x07070707u;
    }
  }
  return intx4{(int)r[0], (int)r[1], (int)r[2], (int)r[3]};
}

// Seven-bit limb `sh/7` of four weights, one per byte.
__device__ __forceinline__ int limb4(const uint4& x, uint32_t sh) {
  const uint32_t b0 = (x.x >> sh) & 0x7Fu, b1 = (x.y >> sh) & 0x7Fu;
  const uint32_t b2 = (x.z >> sh) & 0x7Fu, b3 = (x.w >> sh) & 0x7Fu;
  return (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
}

template <int KB, bool QJL, int VB, bool VLM>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Shared by the 4 waves: the rotated query rows (each wave rotates one head),
  // their QJL projections and the codebooks.  Rows are padded by 4 words so the
  // 4 heads' 16-byte reads fall in different banks.
  __shared__ __align__(16) float q_sh[4][kDim + 4];
  __shared__ __align__(16) float p_sh[QJL ? 4 : 1][kDim + 4];
  __shared__ __align__(16) float kcb[16];
  __shared__ float vcb[16];
  // per wave and head, the 64 tokens' value weights: fp32 (Lloyd-Max values) or
  // the fixed-point integers fed to the int8 MFMA (uniform values)
  __shared__ __align__(16) uint32_t wT[4][4][68];
  __shared__ float part_ml[4][4][2];
  __shared__ __align__(16) float part_o[4][4][kDim];

  const int G = a.group;
  int seq_len = a.seq_lens[b];
  seq_len = max(0, min(seq_len, min(a.max_seq, 16 * a.max_blocks)));
  if (a.num_blocks <= 0) seq_len = 0;     // no page exists: every block id is absent
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = tile_begin + a.tiles_per_split;
  const int tok_end = min(seq_len, tile_end * 64);
  const int64_t head_stride = a.f.page_bytes;
  const int64_t blk_stride = head_stride * a.hkv;
  uint32_t (&wt)[4][68] = wT[wave];

  // Prologue: the block ids of the wave's pages (lane 4k + pg: page pg of the
  // wave's k-th tile; at most 16 tiles per wave since tiles_per_split <= 64) and
  // the query row of head `wave` are fetched together; the first tile's loads
  // are issued before the query is rotated so that their latency overlaps the
  // rotation and the one work-group barrier.
  int blk_reg = -1;
  {
    const int tl = tile_begin + wave + 4 * (lane >> 2);
    const int page = tl * 4 + (lane & 3);
    if (tl < tile_end && page * 16 < tok_end) {
      const int raw = a.block_tables[(int64_t)b * a.max_blocks + page];
      blk_reg = (raw < 0 || (int64_t)raw >= a.num_blocks) ? -1 : raw;
    }
  }
  if (wave == 0 && lane < 16) kcb[lane] = a.c->kc[lane];
  if (VLM && wave == 1 && lane < 16) vcb[lane] = a.c->vc[lane];
  float qx0 = 0.f, qx1 = 0.f;
  if (wave < G) {
    const int64_t qo = ((int64_t)b * a.hq + (int64_t)kvh * G + wave) * kDim + 2 * lane;
    if (a.q_dtype == TQ_BF16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + qo);
      qx0 = bf16lo(w);
      qx1 = bf16hi(w);
    } else {
      const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qo);
      qx0 = f.x;
      qx1 = f.y;
    }
  }
  const float sg0 = a.c->signs[2 * lane], sg1 = a.c->signs[2 * lane + 1];

  TileRegs<KB, VB> nx;
  uint4 vp[VB == 3 ? 8 : 4];     // Lloyd-Max values: byte planes of coordinates 2*lane, 2*lane+1
  uint4 vq[VB];                  // uniform values: the planes of coordinates 8j..8j+7 of page lane/16
  int tile = tile_begin + wave;
  if (tile < tile_end && tile * 64 < tok_end) {
    const int blk = lane_block(blk_reg, 0, lane);
    load_tile<KB, QJL, VB, VLM>(nx, a, blk, kvh, lane, blk_stride, head_stride);
    if constexpr (VLM) load_value_planes<VB>(vp, a, pages_of(blk_reg, 0), kvh, lane, blk_stride, head_stride);
    else load_value_group<VB>(vq, a, blk, kvh, lane, blk_stride, head_stride);
  }

  // Rotate query head `wave`: q'' = log2(e) * scale * H(s*q)/sqrt(d), so that the
  // logits come out in base-2 units for exp2.  Heads >= G stay zero.
  {
    float x0 = qx0 * sg0, x1 = qx1 * sg1;
    const float s0 = x0 + x1, d0 = x0 - x1;
    x0 = s0;
    x1 = d0;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(x0, m), p1 = __shfl_xor(x1, m);
      const bool upper = (lane & m) != 0;
      x0 = upper ? p0 - x0 : x0 + p0;
      x1 = upper ? p1 - x1 : x1 + p1;
    }
    const float f = a.scale * kInvSqrtDim * kLog2e;
    q_sh[wave][2 * lane] = x0 * f;
    q_sh[wave][2 * lane + 1] = x1 * f;
    if constexpr (QJL) {
      // p'' = coef * S q''  (coef = sqrt(pi/2)/m): lane computes rows 2*lane, 2*lane+1
      wave_sync_lds();
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
      for (int k = 0; k < kDim; ++k) {
        const float2 sv = *reinterpret_cast<const float2*>(&a.c->St[k * kDim + 2 * lane]);
        const float qk = q_sh[wave][k];
        acc0 = fmaf(sv.x, qk, acc0);
        acc1 = fmaf(sv.y, qk, acc1);
      }
      p_sh[wave][2 * lane] = acc0 * a.qjl_coef;
      p_sh[wave][2 * lane + 1] = acc1 * a.qjl_coef;
    }
  }
  __syncthreads();

  float m_run[4], l_lane[4], s_lane[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
    s_lane[h] = 0.f;
  }
  // Uniform values: lane l accumulates head l/16, coordinates 8(l%16) + m.
  float O[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) O[m] = 0.f;
  // Lloyd-Max values: rows = heads, columns = coordinates 2*lane, 2*lane+1.
  floatx4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = O0, O2 = O0, O3 = O0;
  const int vsh = (VB == 2) ? 4 * (lane & 1) : (VB == 3) ? ((6 * lane) & 7) : 0;
  const char* cbf = reinterpret_cast<const char*>(&kcb[0]);
  const int ho = lane >> 4;                              // head of this lane's value outputs

  for (int k = 0; tile < tile_end && tile * 64 < tok_end; tile += 4, ++k) {
    const int t = tile * 64 + lane;
    const bool has_next = tile + 4 < tile_end && (tile + 4) * 64 < tok_end;
    const bool valid = t < tok_end && lane_block(blk_reg, k, lane) >= 0;
    const int nblk = lane_block(blk_reg, k + 1, lane);
    // masked lanes may have read another page: their scalars must not reach a sum
    const float knorm = nx.knorm, kres = nx.kres;
    const float va = valid ? nx.va : 0.f, vb = valid ? nx.vb : 0.f;

    // Logits: rows = 4 query heads, columns = this lane's token, one coordinate per
    // MFMA; two independent accumulators keep the matrix pipe busy.
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
    if constexpr (KB == 4) {
      // Two masks per 32-bit word put its eight codes, multiplied by 4 (the table
      // stride), into byte lanes; each code then costs one byte extract.
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t e = (nx.kw[j] << 2) & 0x3C3C3C3Cu;   // codes 8j, 8j+2, 8j+4, 8j+6
        uint32_t o = (nx.kw[j] >> 2) & 0x3C3C3C3Cu;   // codes 8j+1, 8j+3, 8j+5, 8j+7
        // keep the two masked words: folding the masks into each byte extract
        // would cost two instructions per code instead of one
        asm volatile("" : "+v"(e), "+v"(o));
        const float4 qa = *reinterpret_cast<const float4*>(&q_sh[lane & 3][8 * j]);
        const float4 qb = *reinterpret_cast<const float4*>(&q_sh[lane & 3][8 * j + 4]);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.x, *(const float*)(cbf + (e & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.y, *(const float*)(cbf + (o & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.z, *(const float*)(cbf + ((e >> 8) & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.w, *(const float*)(cbf + ((o >> 8) & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.x, *(const float*)(cbf + ((e >> 16) & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.y, *(const float*)(cbf + ((o >> 16) & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.z, *(const float*)(cbf + (e >> 24)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.w, *(const float*)(cbf + (o >> 24)), c1, 0, 0, 0);
        if ((j & 1) == 1) __builtin_amdgcn_sched_barrier(0);   // bound the look-ups in flight
      }
    } else {
#pragma unroll
      for (int i = 0; i < kDim; i += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&q_sh[lane & 3][i]);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.x, *(const float*)(cbf + (get_code<KB>(nx.kw, i) << 2)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.y, *(const float*)(cbf + (get_code<KB>(nx.kw, i + 1) << 2)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.z, *(const float*)(cbf + (get_code<KB>(nx.kw, i + 2) << 2)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.w, *(const float*)(cbf + (get_code<KB>(nx.kw, i + 3) << 2)), c1, 0, 0, 0);
        if ((i & 15) == 12) __builtin_amdgcn_sched_barrier(0);
      }
    }
    floatx4 acc = c0 + c1;
    floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QJL) {
      floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0;
      const uint32_t sgw[4] = {nx.sg.x, nx.sg.y, nx.sg.z, nx.sg.w};
#pragma unroll
      for (int i = 0; i < kDim; i += 2) {
        const float2 p2 = *reinterpret_cast<const float2*>(&p_sh[lane & 3][i]);
        const float s0 = ((sgw[i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
        const float s1 = ((sgw[(i + 1) >> 5] >> ((i + 1) & 31)) & 1u) ? 1.f : -1.f;
        d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.x, s0, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.y, s1, d1, 0, 0, 0);
      }
      acc2 = d0 + d1;
    }
    // The key row is consumed: fetch the next tile while this one finishes.
    if (has_next) load_tile<KB, QJL, VB, VLM>(nx, a, nblk, kvh, lane, blk_stride, head_stride);

    float lg[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v = knorm * acc[h];
      if (QJL) v = fmaf(kres, acc2[h], v);
      lg[h] = valid ? v : -INFINITY;
    }
    if (a.logits != nullptr && valid) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (h < G) a.logits[((int64_t)b * a.hq + (int64_t)kvh * G + h) * a.max_seq + t] = lg[h] * kLn2;
    }
    // Online softmax (base 2): the running max is wave-uniform, sums stay per lane;
    // the accumulators are rescaled only when a head's max moved.
    float mnew[4] = {lg[0], lg[1], lg[2], lg[3]};
    float smax = vb;                        // largest value scale of the tile (masked lanes: 0)
    wave_max5(mnew[0], mnew[1], mnew[2], mnew[3], smax);
    bool moved = false;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      mnew[h] = fmaxf(m_run[h], mnew[h]);
      moved = moved || (mnew[h] != m_run[h]);
    }
    if (moved) {
      float al[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        al[h] = (mnew[h] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[h] - mnew[h]);
        l_lane[h] *= al[h];
        s_lane[h] *= al[h];
        m_run[h] = mnew[h];
      }
      if constexpr (VLM) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          O0[h] *= al[h];
          O1[h] *= al[h];
          O2[h] *= al[h];
          O3[h] *= al[h];
        }
      } else {
        const float ah = ho == 0 ? al[0] : ho == 1 ? al[1] : ho == 2 ? al[2] : al[3];
#pragma unroll
        for (int m = 0; m < 8; ++m) O[m] *= ah;
      }
    }
    float pr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float ms = (m_run[h] == -INFINITY) ? 0.f : m_run[h];
      pr[h] = __builtin_amdgcn_exp2f(lg[h] - ms);          // 0 for masked tokens
      l_lane[h] += pr[h];
      if (!VLM) s_lane[h] = fmaf(pr[h], va, s_lane[h]);
    }
    if constexpr (VLM) {
#pragma unroll
      for (int h = 0; h < 4; ++h) wt[h][lane] = __float_as_uint(pr[h] * va);
      wave_sync_lds();
      // Values: rows = 4 heads, columns = coordinates 2*lane / 2*lane+1, one token per
      // MFMA; even and odd tokens go to separate accumulators.
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int tt = pg * 16 + 4 * kk;
          const uint4 wu = *reinterpret_cast<const uint4*>(&wt[lane & 3][tt]);
          const float4 w4 = make_float4(__uint_as_float(wu.x), __uint_as_float(wu.y), __uint_as_float(wu.z),
                                        __uint_as_float(wu.w));
          uint32_t lo, hi;
          uint32_t x1 = 0u;
          if constexpr (VB == 3) x1 = u4get(vp[4 + pg], kk);
          value_nibbles<VB>(u4get(vp[pg], kk), x1, vsh, lo, hi);
          float b0[4], b1[4];
          b0[0] = vcb[lo & 0xFF]; b0[1] = vcb[(lo >> 8) & 0xFF]; b0[2] = vcb[(lo >> 16) & 0xFF]; b0[3] = vcb[lo >> 24];
          b1[0] = vcb[hi & 0xFF]; b1[1] = vcb[(hi >> 8) & 0xFF]; b1[2] = vcb[(hi >> 16) & 0xFF]; b1[3] = vcb[hi >> 24];
          O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.x, b0[0], O0, 0, 0, 0);
          O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.x, b1[0], O1, 0, 0, 0);
          O2 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.y, b0[1], O2, 0, 0, 0);
          O3 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.y, b1[1], O3, 0, 0, 0);
          O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.z, b0[2], O0, 0, 0, 0);
          O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.z, b1[2], O1, 0, 0, 0);
          O2 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.w, b0[3], O2, 0, 0, 0);
          O3 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.w, b1[3], O3, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep one page's operands live at a time
      }
      if (has_next) load_value_planes<VB>(vp, a, pages_of(blk_reg, k + 1), kvh, lane, blk_stride, head_stride);
    } else {
      // Uniform values, o_h += sum_t p_t (min_t + scale_t * code_t): the min part is
      // a per-head scalar (s_lane); the code part is an exact integer product.  The
      // weights p_t * scale_t become fixed-point integers on a grid shared by the
      // tile, 2^(E-27) with 2^E just above the tile's largest scale (p <= 1), split
      // into four 7-bit limbs: rows of the 16x16x64 int8 MFMA are (head, limb),
      // columns 16 coordinates, and K the tile's 64 tokens.
      const int E = __builtin_amdgcn_frexp_expf(smax);
      const float vbs = ldexpf(vb, 27 - E);
#pragma unroll
      for (int h = 0; h < 4; ++h) wt[h][lane] = (uint32_t)fmaf(pr[h], vbs, 0.5f);   // round to nearest
      wave_sync_lds();
      // A operand: row lane%16 = (head (lane/4)%4, limb lane%4), tokens 16g..16g+15
      // of page g = lane/16, one per byte.
      const uint4* wsrc = reinterpret_cast<const uint4*>(&wt[(lane >> 2) & 3][16 * (lane >> 4)]);
      const uint32_t lsh = 7u * (uint32_t)(lane & 3);
      const intx4 A = {limb4(wsrc[0], lsh), limb4(wsrc[1], lsh), limb4(wsrc[2], lsh), limb4(wsrc[3], lsh)};
      const float bsc = ldexpf(1.f, E - 27);
      const intx4 zero = {0, 0, 0, 0};
#define TQ_PV(M)                                                                                   \
      {                                                                                            \
        const intx4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, value_codes<VB, M>(vq), zero, 0, 0, 0); \
        const uint32_t u = (uint32_t)d[0] + ((uint32_t)d[1] << 7) + ((uint32_t)d[2] << 14);        \
        O[M] = fmaf(fmaf((float)d[3], 2097152.f, (float)u), bsc, O[M]);                             \
      }
      TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
      if (has_next) load_value_group<VB>(vq, a, nblk, kvh, lane, blk_stride, head_stride);
    }
    wave_sync_lds();
  }

  // Per-wave totals, then merge the 4 waves of the work-group.
  float tot[8] = {l_lane[0], l_lane[1], l_lane[2], l_lane[3], s_lane[0], s_lane[1], s_lane[2], s_lane[3]};
  wave_sum8(tot);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      part_ml[wave][h][0] = m_run[h];
      part_ml[wave][h][1] = tot[h];
    }
  }
  if constexpr (VLM) {
    O0 += O2;
    O1 += O3;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      part_o[wave][h][2 * lane] = O0[h];
      part_o[wave][h][2 * lane + 1] = O1[h];
    }
  } else {
    const float sh = ho == 0 ? tot[4] : ho == 1 ? tot[5] : ho == 2 ? tot[6] : tot[7];
    float4* dst = reinterpret_cast<float4*>(&part_o[wave][ho][8 * (lane & 15)]);
    dst[0] = make_float4(O[0] + sh, O[1] + sh, O[2] + sh, O[3] + sh);
    dst[1] = make_float4(O[4] + sh, O[5] + sh, O[6] + sh, O[7] + sh);
  }
  __syncthreads();
  // Merge the 4 waves: thread (head h = wave, coordinates 2*lane, 2*lane+1).
  const int h = wave;
  float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
  if (h < G) {
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, part_ml[w][h][0]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = part_ml[w][h][0];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = fmaf(f, part_ml[w][h][1], L);
      o0 = fmaf(f, part_o[w][h][2 * lane], o0);
      o1 = fmaf(f, part_o[w][h][2 * lane + 1], o1);
    }
  }
  if (a.splits > 1) {
    // Publish this split's partial; the last work-group of the (sequence, kv head)
    // to arrive merges all splits (log-sum-exp) and writes the output.  Partials
    // are written and read with agent-scope (device-coherent) accesses, so no
    // cache-wide write-back or invalidate is needed around the arrival counter.
    if (h < G) {
      float* dst = a.ws + ((((int64_t)b * a.hkv + kvh) * a.splits + split) * 4 + h) * (2 + kDim);
      if (lane == 0) {
        store_agent(dst, M);
        store_agent(dst + 1, L);
      }
      store_agent(dst + 2 + 2 * lane, o0);
      store_agent(dst + 3 + 2 * lane, o1);
    }
    __builtin_amdgcn_s_waitcnt(0);            // every store of this thread has completed
    __syncthreads();
    __shared__ int last;
    if (tid == 0) {
      // wraps back to 0 after `splits` arrivals, so the counter is left zero
      const unsigned prev = __builtin_amdgcn_atomic_inc32(a.counters + (int64_t)b * a.hkv + kvh,
                                                         (unsigned)(a.splits - 1), __ATOMIC_RELAXED, "agent");
      last = prev == (unsigned)(a.splits - 1);
    }
    __syncthreads();
    if (!last) return;
    M = -INFINITY;
    L = o0 = o1 = 0.f;
    if (h < G) {
      const int64_t stride = 4 * (2 + kDim);
      const float* src = a.ws + (((int64_t)b * a.hkv + kvh) * a.splits * 4 + h) * (2 + kDim);
      for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, load_agent(src + sp * stride));
      for (int sp = 0; sp < a.splits; ++sp) {
        const float ms = load_agent(src + sp * stride);
        if (ms != -INFINITY) {
          const float f = __builtin_amdgcn_exp2f(ms - M);
          L = fmaf(f, load_agent(src + sp * stride + 1), L);
          o0 = fmaf(f, load_agent(src + sp * stride + 2 + 2 * lane), o0);
          o1 = fmaf(f, load_agent(src + sp * stride + 3 + 2 * lane), o1);
        }
      }
    }
  }
  float r0 = L > 0.f ? o0 / L : 0.f;
  float r1 = L > 0.f ? o1 / L : 0.f;
  if constexpr (VLM) {
    // Lloyd-Max values were accumulated in the rotated basis: o = diag(s) H o' / sqrt(d).
    float* buf = &part_o[0][0][0] + h * kDim;
    __syncthreads();
    buf[2 * lane] = r0;
    buf[2 * lane + 1] = r1;
    __syncthreads();
#pragma unroll
    for (int len = 1; len < kDim; len <<= 1) {
      const int c0 = 2 * lane, c1 = 2 * lane + 1;
      const float m0 = buf[c0], p0 = buf[c0 ^ len], m1 = buf[c1], p1 = buf[c1 ^ len];
      __syncthreads();
      buf[c0] = (c0 & len) ? p0 - m0 : m0 + p0;
      buf[c1] = (c1 & len) ? p1 - m1 : m1 + p1;
      __syncthreads();
    }
    r0 = buf[2 * lane] * a.c->signs[2 * lane] * kInvSqrtDim;
    r1 = buf[2 * lane + 1] * a.c->signs[2 * lane + 1] * kInvSqrtDim;
  }
  if (h < G) {
    float2* o = reinterpret_cast<float2*>(a.out + ((int64_t)b * a.hq + (int64_t)kvh * G + h) * kDim);
    o[lane] = make_float2(r0, r1);
  }
}

namespace {

template <int KB, bool QJL, int VB>
hipError_t decode_v(const DecodeArgs& a, int val_mode, hipStream_t s) {
  const dim3 grid((unsigned)a.splits, (unsigned)a.hkv, (unsigned)a.batch);
  if (val_mode == TQ_VAL_LLOYD) hipLaunchKernelGGL((decode_kernel<KB, QJL, VB, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((decode_kernel<KB, QJL, VB, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t decode_vb(const DecodeArgs& a, int val_bits, int val_mode, hipStream_t s) {
  switch (val_bits) {
    case 2: return decode_v<KB, QJL, 2>(a, val_mode, s);
    case 3: return decode_v<KB, QJL, 3>(a, val_mode, s);
    case 4: return decode_v<KB, QJL, 4>(a, val_mode, s);
  }
  return hipErrorInvalidValue;
}

template <int KB, bool QJL>
const void* kernel_vb(int val_bits, int val_mode) {
  const bool lm = val_mode == TQ_VAL_LLOYD;
  switch (val_bits) {
    case 2: return lm ? (const void*)decode_kernel<KB, QJL, 2, true> : (const void*)decode_kernel<KB, QJL, 2, false>;
    case 3: return lm ? (const void*)decode_kernel<KB, QJL, 3, true> : (const void*)decode_kernel<KB, QJL, 3, false>;
    case 4: return lm ? (const void*)decode_kernel<KB, QJL, 4, true> : (const void*)decode_kernel<KB, QJL, 4, false>;
  }
  return nullptr;
}

}  // namespace

const void* decode_kernel_ptr(int key_bits, int key_mode, int val_bits, int val_mode) {
  const bool qjl = key_mode == TQ_KEY_LLOYD_QJL;
  switch (key_bits) {
    case 2: return qjl ? kernel_vb<2, true>(val_bits, val_mode) : kernel_vb<2, false>(val_bits, val_mode);
    case 3: return qjl ? kernel_vb<3, true>(val_bits, val_mode) : kernel_vb<3, false>(val_bits, val_mode);
    case 4: return qjl ? kernel_vb<4, true>(val_bits, val_mode) : kernel_vb<4, false>(val_bits, val_mode);
  }
  return nullptr;
}

hipError_t launch_decode(const DecodeArgs& a, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s) {
  const bool qjl = key_mode == TQ_KEY_LLOYD_QJL;
  switch (key_bits) {
    case 2: return qjl ? decode_vb<2, true>(a, val_bits, val_mode, s) : decode_vb<2, false>(a, val_bits, val_mode, s);
    case 3: return qjl ? decode_vb<3, true>(a, val_bits, val_mode, s) : decode_vb<3, false>(a, val_bits, val_mode, s);
    case 4: return qjl ? decode_vb<4, true>(a, val_bits, val_mode, s) : decode_vb<4, false>(a, val_bits, val_mode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
