// Decode attention over the packed cache for gfx950 (one launch, split merge included).
//
// Sources (page and section): issoh.co.jp "TurboQuantとは？…", the section on
// where the zero-loss claim comes from (logits against 4-bit keys are the part
// that is sped up); ai-navigate-news turboquant-vllm write-up (attention has to
// be fused over the compressed cache); lilting.ch TurboQuant article, QJL section
// (query kept in full precision, projected with the same S; corrected score).
//
// One work-group per (split of the context, kv head, sequence); each wave owns
// 64-token tiles.  Lane l holds token l's packed key row; codes become centroids
// through a 16-entry LDS table and are contracted with the group's 4 rotated
// query heads on the fp32 4x4x1 (16-block) MFMA, which keeps exact fp32
// products.  The online softmax runs per lane; value codes staged in LDS are
// contracted with the softmax weights on the same MFMA.  Per-split partials
// (max, sum, 128 outputs) go to the workspace; the last work-group of each
// (sequence, kv head) to finish, found with a self-resetting arrival counter,
// merges them by log-sum-exp and writes the output.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

// ---------------------------------------------------------------------------
// Decode attention.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
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

// Codes of coordinates 2*lane and 2*lane+1 of one value row (VB bits each).
template <int VB>
__device__ __forceinline__ uint32_t value_code_pair(const uint8_t* row, int lane) {
  if constexpr (VB == 4) {
    return row[lane];
  } else if constexpr (VB == 2) {
    return (row[lane >> 1] >> (4 * (lane & 1))) & 0xfu;
  } else {
    const int bit = 6 * lane, wi = bit >> 5, sh = bit & 31;
    const uint32_t* r32 = reinterpret_cast<const uint32_t*>(row);
    uint32_t v = r32[wi] >> sh;
    if (sh > 26) v |= r32[wi + 1] << (32 - sh);
    return v & 0x3fu;
  }
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

template <int KB, int VB>
struct TileRegs {
  uint4 kr[KB];
  uint4 vr[VB];
  float knorm, va, vb, kres;
  uint4 sg;
};

// Loads of one 64-token tile (4 pages of one kv head).
template <int KB, bool QJL, int VB, bool VLM>
__device__ __forceinline__ TileRegs<KB, VB> load_tile(const DecodeArgs& a, const int* blk_lds, int tile, int tile_begin,
                                                      int tok_end, int kvh, int lane, int64_t blk_stride,
                                                      int64_t head_stride) {
  constexpr int KROW = kDim * KB / 8;
  constexpr int VROW = kDim * VB / 8;
  TileRegs<KB, VB> r;
  const int t = tile * 64 + lane;
  const int blk = blk_lds[(tile - tile_begin) * 4 + (lane >> 4)];
  const bool valid = t < tok_end && blk >= 0;
  const uint8_t* page = a.cache + (valid ? (int64_t)blk * blk_stride + kvh * head_stride : 0);
  const int so = t & 15;
  r.knorm = 0.f;
  r.va = 0.f;
  r.vb = 0.f;
  r.kres = 0.f;
  r.sg = make_uint4(0u, 0u, 0u, 0u);
  if (valid) {
    r.knorm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
    r.va = reinterpret_cast<const float*>(page + a.f.vmin)[so];
    if (!VLM) r.vb = reinterpret_cast<const float*>(page + a.f.vscale)[so];
    if (QJL) {
      r.sg = reinterpret_cast<const uint4*>(page + a.f.ksigns)[so];
      r.kres = reinterpret_cast<const float*>(page + a.f.kres)[so];
    }
  }
#pragma unroll
  for (int it = 0; it < KB; ++it) {
    const int idx = it * 64 + lane;
    const int pg = idx / KROW, ch = idx - pg * KROW;
    const int pblk = blk_lds[(tile - tile_begin) * 4 + pg];
    r.kr[it] = make_uint4(0u, 0u, 0u, 0u);
    if (pblk >= 0)
      r.kr[it] = *reinterpret_cast<const uint4*>(a.cache + (int64_t)pblk * blk_stride + kvh * head_stride +
                                                 a.f.kcodes + ch * 16);
  }
#pragma unroll
  for (int it = 0; it < VB; ++it) {
    const int idx = it * 64 + lane;
    const int pg = idx / VROW, ch = idx - pg * VROW;
    const int pblk = blk_lds[(tile - tile_begin) * 4 + pg];
    r.vr[it] = make_uint4(0u, 0u, 0u, 0u);
    if (pblk >= 0)
      r.vr[it] = *reinterpret_cast<const uint4*>(a.cache + (int64_t)pblk * blk_stride + kvh * head_stride +
                                                 a.f.vcodes + ch * 16);
  }
  return r;
}

template <int KB, bool QJL, int VB, bool VLM>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int KROW = kDim * KB / 8;   // bytes of one key row
  constexpr int VROW = kDim * VB / 8;   // bytes of one value row
  // LDS stride of a staged key row: odd number of 16-byte chunks -> conflict-free row reads
  constexpr int KSTRIDE = ((KROW / 16) % 2 == 0) ? KROW + 16 : KROW;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // rows padded by 4 floats so the 4 heads' 16-byte reads fall in different banks
  __shared__ __align__(16) float q_lds[4][kDim + 4];
  __shared__ __align__(16) float p_lds[QJL ? 4 : 1][kDim + 4];
  __shared__ float kcb[16];
  __shared__ float vcb[16];
  __shared__ int blk_lds[kMaxPagesPerSplit];
  // Per-wave staging of the current tile: first its key rows (padded rows), then,
  // once every lane holds its row, its value codes (4 pages x 16 rows).  Reused
  // for the per-wave partial outputs at the end.
  constexpr int STAGE = (64 * KSTRIDE > 64 * VROW) ? 64 * KSTRIDE : 64 * VROW;
  constexpr int STAGE_ALL = (4 * STAGE > 4 * 4 * kDim * 4) ? 4 * STAGE : 4 * 4 * kDim * 4;
  __shared__ __align__(16) uint8_t stage[STAGE_ALL];
  __shared__ __align__(16) float wT[4][4][68];      // softmax weight x scale: [wave][head][token]
  __shared__ float part_ml[4][4][2];

  if (tid < 16) {
    kcb[tid] = a.c->kc[tid];
    vcb[tid] = a.c->vc[tid];
  }
  const int G = a.group;
  int seq_len = a.seq_lens[b];
  seq_len = max(0, min(seq_len, min(a.max_seq, 16 * a.max_blocks)));
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = tile_begin + a.tiles_per_split;
  const int tok_end = min(seq_len, tile_end * 64);
  const int64_t head_stride = a.f.page_bytes;
  const int64_t blk_stride = head_stride * a.hkv;

  // Block ids of this split's pages (-1: absent or out of range).
  for (int i = tid; i < a.tiles_per_split * 4; i += 256) {
    const int pg = tile_begin * 4 + i;
    int blk = -1;
    if (pg * 16 < tok_end) {
      blk = a.block_tables[(int64_t)b * a.max_blocks + pg];
      if (blk < 0 || (int64_t)blk >= a.num_blocks) blk = -1;
    }
    blk_lds[i] = blk;
  }

  // Query prologue: wave w rotates q head kvh*G + w once: q'' = scale * H(s*q)/sqrt(d).
  {
    float x0 = 0.f, x1 = 0.f;
    if (wave < G) {
      const int64_t qo = ((int64_t)b * a.hq + (int64_t)kvh * G + wave) * kDim + 2 * lane;
      if (a.q_dtype == TQ_BF16) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + qo);
        x0 = bf16lo(w);
        x1 = bf16hi(w);
      } else {
        const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qo);
        x0 = f.x;
        x1 = f.y;
      }
      x0 *= a.c->signs[2 * lane];
      x1 *= a.c->signs[2 * lane + 1];
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
      const float f = a.scale * kInvSqrtDim;
      x0 *= f;
      x1 *= f;
    }
    q_lds[wave][2 * lane] = x0;
    q_lds[wave][2 * lane + 1] = x1;
  }
  __syncthreads();
  if constexpr (QJL) {
    // p'' = coef * S q''  (coef = sqrt(pi/2)/m)
    for (int idx = tid; idx < 4 * kDim; idx += 256) {
      const int hh = idx >> 7, m = idx & (kDim - 1);
      float acc = 0.f;
#pragma unroll 8
      for (int k = 0; k < kDim; ++k) acc = fmaf(a.c->St[k * kDim + m], q_lds[hh][k], acc);
      p_lds[hh][m] = acc * a.qjl_coef;
    }
    __syncthreads();
  }

  float m_run[4], l_lane[4], s_lane[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
    s_lane[h] = 0.f;
  }
  floatx4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = O0, O2 = O0, O3 = O0;

  // Registers of the tile being loaded (prefetched one tile ahead).  Key and value
  // codes are fetched as contiguous 16-byte chunks of each page (coalesced) and
  // staged through LDS; the per-token scalars are read by the token's lane.
  TileRegs<KB, VB> nx;
  __syncthreads();   // blk_lds ready

  int tile = tile_begin + wave;
  if (tile < tile_end && tile * 64 < tok_end)
    nx = load_tile<KB, QJL, VB, VLM>(a, blk_lds, tile, tile_begin, tok_end, kvh, lane, blk_stride, head_stride);
  for (; tile < tile_end && tile * 64 < tok_end; tile += 4) {
    const int t = tile * 64 + lane;
    const bool valid = t < tok_end && blk_lds[(tile - tile_begin) * 4 + (lane >> 4)] >= 0;
    uint8_t* st = stage + wave * STAGE;
#pragma unroll
    for (int it = 0; it < KB; ++it) {
      // chunk idx of the tile's key rows: row idx / (KROW/16), chunk idx % (KROW/16)
      const int idx = it * 64 + lane;
      const int row = idx / (KROW / 16), ch = idx - row * (KROW / 16);
      *reinterpret_cast<uint4*>(&st[row * KSTRIDE + ch * 16]) = nx.kr[it];
    }
    wave_sync_lds();
    uint32_t kw[KB * 4];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 u = *reinterpret_cast<const uint4*>(&st[lane * KSTRIDE + j * 16]);
      kw[4 * j] = u.x; kw[4 * j + 1] = u.y; kw[4 * j + 2] = u.z; kw[4 * j + 3] = u.w;
    }
    wave_sync_lds();
#pragma unroll
    for (int it = 0; it < VB; ++it) *reinterpret_cast<uint4*>(&st[(it * 64 + lane) * 16]) = nx.vr[it];

    // Logits: rows = 4 query heads, columns = this lane's token, one coordinate per
    // MFMA; four independent accumulators keep the matrix pipe busy.
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
    for (int i = 0; i < kDim; i += 4) {
      const float4 q4 = *reinterpret_cast<const float4*>(&q_lds[lane & 3][i]);
      c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.x, kcb[get_code<KB>(kw, i)], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.y, kcb[get_code<KB>(kw, i + 1)], c1, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.z, kcb[get_code<KB>(kw, i + 2)], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.w, kcb[get_code<KB>(kw, i + 3)], c1, 0, 0, 0);
    }
    floatx4 acc = c0 + c1;
    floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QJL) {
      floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0;
#pragma unroll
      for (int i = 0; i < kDim; i += 2) {
        const float2 p2 = *reinterpret_cast<const float2*>(&p_lds[lane & 3][i]);
        const uint32_t sgw[4] = {nx.sg.x, nx.sg.y, nx.sg.z, nx.sg.w};
        const float s0 = ((sgw[i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
        const float s1 = ((sgw[(i + 1) >> 5] >> ((i + 1) & 31)) & 1u) ? 1.f : -1.f;
        d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.x, s0, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(p2.y, s1, d1, 0, 0, 0);
      }
      acc2 = d0 + d1;
    }
    const float knorm_c = nx.knorm, va_c = nx.va, vb_c = nx.vb, kres_c = nx.kres;
    // The key row is consumed: fetch the next tile while this one finishes.
    if (tile + 4 < tile_end && (tile + 4) * 64 < tok_end)
      nx = load_tile<KB, QJL, VB, VLM>(a, blk_lds, tile + 4, tile_begin, tok_end, kvh, lane, blk_stride, head_stride);

    float lg[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v = knorm_c * acc[h];
      if (QJL) v = fmaf(kres_c, acc2[h], v);
      lg[h] = valid ? v : -INFINITY;
    }
    if (a.logits != nullptr && valid) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (h < G) a.logits[((int64_t)b * a.hq + (int64_t)kvh * G + h) * a.max_seq + t] = lg[h];
    }
    // Online softmax (running max is wave-uniform; sums stay per lane).
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float mnew = fmaxf(m_run[h], wave_max_dpp(lg[h]));
      float alpha = 1.f, pr = 0.f;
      if (mnew != -INFINITY) {
        alpha = __expf(m_run[h] - mnew);
        pr = valid ? __expf(lg[h] - mnew) : 0.f;
      }
      l_lane[h] = fmaf(l_lane[h], alpha, pr);
      if (!VLM) s_lane[h] = fmaf(s_lane[h], alpha, pr * va_c);
      O0[h] *= alpha;
      O1[h] *= alpha;
      O2[h] *= alpha;
      O3[h] *= alpha;
      m_run[h] = mnew;
      wT[wave][h][lane] = pr * (VLM ? va_c : vb_c);
    }
    wave_sync_lds();
    // Values: rows = 4 heads, columns = coordinates 2*lane / 2*lane+1, one token per
    // MFMA; even and odd tokens go to separate accumulators.
    const uint8_t* vs = st;
#pragma unroll 2
    for (int tt = 0; tt < 64; tt += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&wT[wave][lane & 3][tt]);
      const float wu[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t pair = value_code_pair<VB>(vs + (tt + u) * VROW, lane);
        float b0, b1;
        if (VLM) {
          b0 = vcb[pair & ((1u << VB) - 1u)];
          b1 = vcb[pair >> VB];
        } else {
          b0 = (float)(pair & ((1u << VB) - 1u));
          b1 = (float)(pair >> VB);
        }
        if (u & 1) {
          O2 = __builtin_amdgcn_mfma_f32_4x4x1f32(wu[u], b0, O2, 0, 0, 0);
          O3 = __builtin_amdgcn_mfma_f32_4x4x1f32(wu[u], b1, O3, 0, 0, 0);
        } else {
          O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(wu[u], b0, O0, 0, 0, 0);
          O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(wu[u], b1, O1, 0, 0, 0);
        }
      }
    }
    wave_sync_lds();
  }
  O0 += O2;
  O1 += O3;
  float* part_o = reinterpret_cast<float*>(stage);   // [4 waves][4 heads][128]
  __syncthreads();

  // Per-wave totals, then merge the 4 waves of the work-group.
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float lsum = wave_sum(l_lane[h]);
    const float ssum = VLM ? 0.f : wave_sum(s_lane[h]);
    if (lane == 0) {
      part_ml[wave][h][0] = m_run[h];
      part_ml[wave][h][1] = lsum;
    }
    part_o[(wave * 4 + h) * kDim + 2 * lane] = O0[h] + ssum;
    part_o[(wave * 4 + h) * kDim + 2 * lane + 1] = O1[h] + ssum;
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
      o0 = fmaf(f, part_o[(w * 4 + h) * kDim + 2 * lane], o0);
      o1 = fmaf(f, part_o[(w * 4 + h) * kDim + 2 * lane + 1], o1);
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
    float* buf = part_o + h * kDim;      // reuse LDS: [4][128]
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
