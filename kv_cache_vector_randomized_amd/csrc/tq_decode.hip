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
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
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

// Loads of one 64-token tile (4 pages of one kv head).
// Block ids of the 4 pages of one tile (wave-uniform; -1: absent or out of range).
struct TilePages {
  int b[4];
  __device__ __forceinline__ int of_lane(int lane) const {
    const int q = lane >> 4;
    return q == 0 ? b[0] : q == 1 ? b[1] : q == 2 ? b[2] : b[3];
  }
};

// The wave keeps the block ids of all its tiles in one register: lane 4k + pg
// holds page pg of the wave's k-th tile.
__device__ __forceinline__ TilePages pages_of(int blk_reg, int k) {
  TilePages p;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) p.b[pg] = __builtin_amdgcn_readlane(blk_reg, 4 * k + pg);
  return p;
}

template <int KB, bool QJL, int VB, bool VLM>
__device__ __forceinline__ void load_tile(TileRegs<KB, VB>& r, const DecodeArgs& a, const TilePages& tp, int tile,
                                          int tok_end, int kvh, int lane, int64_t blk_stride,
                                          int64_t head_stride) {
  constexpr int KROW = kDim * KB / 8;
  constexpr int VROW = kDim * VB / 8;
  const int t = tile * 64 + lane;
  const int blk = tp.of_lane(lane);
  const bool valid = t < tok_end && blk >= 0;
  const uint8_t* page = a.cache + (valid ? (int64_t)blk * blk_stride + kvh * head_stride : 0);
  const int so = t & 15;
  r.knorm = 0.f;
  r.va = 0.f;
  r.vb = 0.f;
  r.kres = 0.f;
  r.sg = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int j = 0; j < KB * 4; ++j) r.kw[j] = 0u;
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(page + a.f.kcodes + so * KROW);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 u = src[j];
      r.kw[4 * j] = u.x; r.kw[4 * j + 1] = u.y; r.kw[4 * j + 2] = u.z; r.kw[4 * j + 3] = u.w;
    }
    r.knorm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
    r.va = reinterpret_cast<const float*>(page + a.f.vmin)[so];
    if (!VLM) r.vb = reinterpret_cast<const float*>(page + a.f.vscale)[so];
    if (QJL) {
      r.sg = reinterpret_cast<const uint4*>(page + a.f.ksigns)[so];
      r.kres = reinterpret_cast<const float*>(page + a.f.kres)[so];
    }
  }
}

// Value byte plane(s) of this lane's two coordinates for the tile's 4 pages
// (16 tokens per page, one coalesced 16-byte load per page and plane).
template <int VB>
__device__ __forceinline__ void load_value_planes(uint4 (&vp)[VB == 3 ? 8 : 4], const DecodeArgs& a,
                                                  const TilePages& tp, int kvh, int lane, int64_t blk_stride,
                                                  int64_t head_stride) {
  constexpr int VROW = kDim * VB / 8;
  const int p0 = (VB == 4) ? lane : (VB == 2) ? (lane >> 1) : ((6 * lane) >> 3);
  const int p1 = (6 * lane >> 3) + 1 < VROW ? (6 * lane >> 3) + 1 : VROW - 1;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {
    const int pblk = tp.b[pg];
    vp[pg] = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (VB == 3) vp[4 + pg] = make_uint4(0u, 0u, 0u, 0u);
    if (pblk >= 0) {
      const uint8_t* vbase = a.cache + (int64_t)pblk * blk_stride + kvh * head_stride + a.f.vcodes;
      vp[pg] = *reinterpret_cast<const uint4*>(vbase + p0 * 16);
      if constexpr (VB == 3) vp[4 + pg] = *reinterpret_cast<const uint4*>(vbase + p1 * 16);
    }
  }
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

template <int KB, bool QJL, int VB, bool VLM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Each wave owns its copy of the rotated query rows and the codebooks, so the
  // waves never wait for each other before the final merge.  Rows are padded by
  // 4 floats so the 4 heads' 16-byte reads fall in different banks.
  __shared__ __align__(16) float q_all[4][4][kDim + 4];
  __shared__ __align__(16) float p_all[QJL ? 4 : 1][QJL ? 4 : 1][kDim + 4];
  __shared__ float kcb_all[4][16];
  __shared__ float vcb_all[4][16];
  __shared__ __align__(16) float wT[4][4][68];      // softmax weight x scale: [wave][head][token]
  __shared__ float part_ml[4][4][2];
  __shared__ __align__(16) float part_o[4][4][kDim];

  const int G = a.group;
  int seq_len = a.seq_lens[b];
  seq_len = max(0, min(seq_len, min(a.max_seq, 16 * a.max_blocks)));
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = tile_begin + a.tiles_per_split;
  const int tok_end = min(seq_len, tile_end * 64);
  const int64_t head_stride = a.f.page_bytes;
  const int64_t blk_stride = head_stride * a.hkv;

  float (&q_lds)[4][kDim + 4] = q_all[wave];
  float (&p_lds)[QJL ? 4 : 1][kDim + 4] = p_all[QJL ? wave : 0];
  float* kcb = kcb_all[wave];
  float* vcb = vcb_all[wave];

  // Prologue (per wave, no work-group barrier): the block ids of the wave's
  // pages (lane 4k + pg: page pg of the wave's k-th tile; at most 16 tiles per
  // wave since tiles_per_split <= 64) and the query rows are fetched together;
  // the first tile's loads are issued before the query is rotated so that their
  // latency overlaps the rotation.
  int blk_reg = -1;
  {
    const int tl = tile_begin + wave + 4 * (lane >> 2);
    const int page = tl * 4 + (lane & 3);
    if (tl < tile_end && page * 16 < tok_end) {
      const int raw = a.block_tables[(int64_t)b * a.max_blocks + page];
      blk_reg = (raw < 0 || (int64_t)raw >= a.num_blocks) ? -1 : raw;
    }
  }
  if (lane < 16) {
    kcb[lane] = a.c->kc[lane];
    vcb[lane] = a.c->vc[lane];
  }
  float qx[4][2], sg0 = 0.f, sg1 = 0.f;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    qx[hh][0] = qx[hh][1] = 0.f;
    if (hh < G) {
      const int64_t qo = ((int64_t)b * a.hq + (int64_t)kvh * G + hh) * kDim + 2 * lane;
      if (a.q_dtype == TQ_BF16) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + qo);
        qx[hh][0] = bf16lo(w);
        qx[hh][1] = bf16hi(w);
      } else {
        const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qo);
        qx[hh][0] = f.x;
        qx[hh][1] = f.y;
      }
    }
  }
  sg0 = a.c->signs[2 * lane];
  sg1 = a.c->signs[2 * lane + 1];

  TileRegs<KB, VB> nx;
  uint4 vp[VB == 3 ? 8 : 4];
  int tile = tile_begin + wave;
  if (tile < tile_end && tile * 64 < tok_end) {
    const TilePages tp = pages_of(blk_reg, 0);
    load_tile<KB, QJL, VB, VLM>(nx, a, tp, tile, tok_end, kvh, lane, blk_stride, head_stride);
    load_value_planes<VB>(vp, a, tp, kvh, lane, blk_stride, head_stride);
  }

  // Rotate the group's query heads once: q'' = scale * H(s*q)/sqrt(d).
  {
    const float f = a.scale * kInvSqrtDim;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      float x0 = qx[hh][0] * sg0, x1 = qx[hh][1] * sg1;
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
      q_lds[hh][2 * lane] = x0 * f;
      q_lds[hh][2 * lane + 1] = x1 * f;
    }
  }
  wave_sync_lds();
  if constexpr (QJL) {
    // p'' = coef * S q''  (coef = sqrt(pi/2)/m): lane computes rows 2*lane, 2*lane+1
    float acc[4][2];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) acc[hh][0] = acc[hh][1] = 0.f;
#pragma unroll 4
    for (int k = 0; k < kDim; ++k) {
      const float2 sv = *reinterpret_cast<const float2*>(&a.c->St[k * kDim + 2 * lane]);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float qk = q_lds[hh][k];
        acc[hh][0] = fmaf(sv.x, qk, acc[hh][0]);
        acc[hh][1] = fmaf(sv.y, qk, acc[hh][1]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      p_lds[hh][2 * lane] = acc[hh][0] * a.qjl_coef;
      p_lds[hh][2 * lane + 1] = acc[hh][1] * a.qjl_coef;
    }
    wave_sync_lds();
  }

  float m_run[4], l_lane[4], s_lane[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
    s_lane[h] = 0.f;
  }
  floatx4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = O0, O2 = O0, O3 = O0;
  const int vsh = (VB == 2) ? 4 * (lane & 1) : (VB == 3) ? ((6 * lane) & 7) : 0;

  for (int k = 0; tile < tile_end && tile * 64 < tok_end; tile += 4, ++k) {
    const int t = tile * 64 + lane;
    const TilePages tp = pages_of(blk_reg, k);
    const bool valid = t < tok_end && tp.of_lane(lane) >= 0;
    const float knorm = nx.knorm, va = nx.va, vb = nx.vb, kres = nx.kres;

    // Logits: rows = 4 query heads, columns = this lane's token, one coordinate per
    // MFMA; two independent accumulators keep the matrix pipe busy.
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
    const char* cb = reinterpret_cast<const char*>(kcb);
    if constexpr (KB == 4) {
      // Two masks per 32-bit word put its eight codes, already multiplied by 4 (the
      // table stride), into byte lanes; each code then costs one byte extract.
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t e = (nx.kw[j] << 2) & 0x3C3C3C3Cu;   // codes 8j, 8j+2, 8j+4, 8j+6
        const uint32_t o = (nx.kw[j] >> 2) & 0x3C3C3C3Cu;   // codes 8j+1, 8j+3, 8j+5, 8j+7
        const float4 qa = *reinterpret_cast<const float4*>(&q_lds[lane & 3][8 * j]);
        const float4 qb = *reinterpret_cast<const float4*>(&q_lds[lane & 3][8 * j + 4]);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.x, *(const float*)(cb + (e & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.y, *(const float*)(cb + (o & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.z, *(const float*)(cb + ((e >> 8) & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qa.w, *(const float*)(cb + ((o >> 8) & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.x, *(const float*)(cb + ((e >> 16) & 0xFF)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.y, *(const float*)(cb + ((o >> 16) & 0xFF)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.z, *(const float*)(cb + (e >> 24)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qb.w, *(const float*)(cb + (o >> 24)), c1, 0, 0, 0);
        if ((j & 1) == 1) __builtin_amdgcn_sched_barrier(0);   // bound the look-ups in flight
      }
    } else {
#pragma unroll
      for (int i = 0; i < kDim; i += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&q_lds[lane & 3][i]);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.x, *(const float*)(cb + (get_code<KB>(nx.kw, i) << 2)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.y, *(const float*)(cb + (get_code<KB>(nx.kw, i + 1) << 2)), c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.z, *(const float*)(cb + (get_code<KB>(nx.kw, i + 2) << 2)), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.w, *(const float*)(cb + (get_code<KB>(nx.kw, i + 3) << 2)), c1, 0, 0, 0);
      }
    }
    floatx4 acc = c0 + c1;
    floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QJL) {
      floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0;
      const uint32_t sgw[4] = {nx.sg.x, nx.sg.y, nx.sg.z, nx.sg.w};
#pragma unroll
      for (int i = 0; i < kDim; i += 2) {
        const float2 p2 = *reinterpret_cast<const float2*>(&p_lds[lane & 3][i]);
        const float s0 = ((sgw[i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
        const float s1 = ((sgw[(i + 1) >> 5] >> ((i + 1) & 31)) & 1u) ? 1.f : -1.f;
        d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.x, s0, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.y, s1, d1, 0, 0, 0);
      }
      acc2 = d0 + d1;
    }
    // The key row is consumed: fetch the next tile while this one finishes.
    if (tile + 4 < tile_end && (tile + 4) * 64 < tok_end)
      load_tile<KB, QJL, VB, VLM>(nx, a, pages_of(blk_reg, k + 1), tile + 4, tok_end, kvh, lane, blk_stride,
                                  head_stride);

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
        if (h < G) a.logits[((int64_t)b * a.hq + (int64_t)kvh * G + h) * a.max_seq + t] = lg[h];
    }
    // Online softmax: the running max is wave-uniform, sums stay per lane; the
    // accumulators are rescaled only when a head's max moved.
    float mnew[4];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      mnew[h] = fmaxf(m_run[h], wave_max_dpp(lg[h]));
      moved = moved || (mnew[h] != m_run[h]);
    }
    if (moved) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float alpha = (mnew[h] == -INFINITY) ? 1.f : __expf(m_run[h] - mnew[h]);
        l_lane[h] *= alpha;
        s_lane[h] *= alpha;
        O0[h] *= alpha;
        O1[h] *= alpha;
        O2[h] *= alpha;
        O3[h] *= alpha;
        m_run[h] = mnew[h];
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float pr = (valid && m_run[h] != -INFINITY) ? __expf(lg[h] - m_run[h]) : 0.f;
      l_lane[h] += pr;
      if (!VLM) s_lane[h] = fmaf(pr, va, s_lane[h]);
      wT[wave][h][lane] = pr * (VLM ? va : vb);
    }
    wave_sync_lds();
    // Values: rows = 4 heads, columns = coordinates 2*lane / 2*lane+1, one token per
    // MFMA; even and odd tokens go to separate accumulators.
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tt = pg * 16 + 4 * k;
        const float4 w4 = *reinterpret_cast<const float4*>(&wT[wave][lane & 3][tt]);
        uint32_t lo, hi;
        uint32_t x1 = 0u;
        if constexpr (VB == 3) x1 = u4get(vp[4 + pg], k);
        value_nibbles<VB>(u4get(vp[pg], k), x1, vsh, lo, hi);
        float b0[4], b1[4];
        if (VLM) {
          b0[0] = vcb[lo & 0xFF]; b0[1] = vcb[(lo >> 8) & 0xFF]; b0[2] = vcb[(lo >> 16) & 0xFF]; b0[3] = vcb[lo >> 24];
          b1[0] = vcb[hi & 0xFF]; b1[1] = vcb[(hi >> 8) & 0xFF]; b1[2] = vcb[(hi >> 16) & 0xFF]; b1[3] = vcb[hi >> 24];
        } else {
          // byte -> float (v_cvt_f32_ubyte0..3)
          b0[0] = (float)(lo & 0xFF); b0[1] = (float)((lo >> 8) & 0xFF);
          b0[2] = (float)((lo >> 16) & 0xFF); b0[3] = (float)(lo >> 24);
          b1[0] = (float)(hi & 0xFF); b1[1] = (float)((hi >> 8) & 0xFF);
          b1[2] = (float)((hi >> 16) & 0xFF); b1[3] = (float)(hi >> 24);
        }
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
    // value planes of the next tile (its key rows are already on the way)
    if (tile + 4 < tile_end && (tile + 4) * 64 < tok_end)
      load_value_planes<VB>(vp, a, pages_of(blk_reg, k + 1), kvh, lane, blk_stride, head_stride);
    wave_sync_lds();
  }
  O0 += O2;
  O1 += O3;

  // Per-wave totals, then merge the 4 waves of the work-group.
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float lsum = wave_sum(l_lane[h]);
    const float ssum = VLM ? 0.f : wave_sum(s_lane[h]);
    if (lane == 0) {
      part_ml[wave][h][0] = m_run[h];
      part_ml[wave][h][1] = lsum;
    }
    part_o[wave][h][2 * lane] = O0[h] + ssum;
    part_o[wave][h][2 * lane + 1] = O1[h] + ssum;
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
      const float f = (mw == -INFINITY) ? 0.f : __expf(mw - M);
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
          const float f = __expf(ms - M);
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

}  // namespace

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
