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

template <int KB, bool QJL, int VB, bool VLM>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int KROW = kDim * KB / 8;   // bytes of one key row
  constexpr int VROW = kDim * VB / 8;   // bytes of one value row
  constexpr int VCHUNKS = VROW;         // 16-byte chunks of one page's value codes (16 rows)
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float q_lds[4][kDim];
  __shared__ float p_lds[QJL ? 4 : 1][kDim];
  __shared__ float kcb[16];
  __shared__ float vcb[16];
  __shared__ __align__(16) uint8_t vstage[4][4 * 16 * VROW + 16];
  __shared__ float4 wbuf[4][64];
  __shared__ float part_ml[4][4][2];
  __shared__ float part_o[4][4][kDim];

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
  float qreg[kDim];
#pragma unroll
  for (int i = 0; i < kDim; ++i) qreg[i] = q_lds[lane & 3][i];

  float m_run[4], l_lane[4], s_lane[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
    s_lane[h] = 0.f;
  }
  floatx4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = {0.f, 0.f, 0.f, 0.f};
  const int64_t head_stride = a.f.page_bytes;
  const int64_t blk_stride = head_stride * a.hkv;

  for (int tile = tile_begin + wave; tile < tile_end && tile * 64 < tok_end; tile += 4) {
    const int t = tile * 64 + lane;
    bool valid = t < tok_end;
    int blk = valid ? a.block_tables[(int64_t)b * a.max_blocks + (t >> 4)] : -1;
    valid = valid && blk >= 0 && (int64_t)blk < a.num_blocks;
    if (!valid) blk = -1;
    const uint8_t* page = a.cache + (valid ? (int64_t)blk * blk_stride + kvh * head_stride : 0);
    const int so = t & 15;

    uint32_t kw[KB * 4];
    float knorm = 0.f, va = 0.f, vb = 0.f, kres = 0.f;
    uint32_t sg[4] = {0u, 0u, 0u, 0u};
    if (valid) {
      const uint4* src = reinterpret_cast<const uint4*>(page + a.f.kcodes + so * KROW);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const uint4 u = src[j];
        kw[4 * j] = u.x; kw[4 * j + 1] = u.y; kw[4 * j + 2] = u.z; kw[4 * j + 3] = u.w;
      }
      knorm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
      va = reinterpret_cast<const float*>(page + a.f.vmin)[so];
      if (!VLM) vb = reinterpret_cast<const float*>(page + a.f.vscale)[so];
      if (QJL) {
        const uint4 u = reinterpret_cast<const uint4*>(page + a.f.ksigns)[so];
        sg[0] = u.x; sg[1] = u.y; sg[2] = u.z; sg[3] = u.w;
        kres = reinterpret_cast<const float*>(page + a.f.kres)[so];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KB * 4; ++j) kw[j] = 0u;
    }
    // Stage the value codes of the tile's 4 pages in LDS (coalesced 16-byte chunks).
#pragma unroll
    for (int it = 0; it < (4 * VCHUNKS) / 64; ++it) {
      const int idx = it * 64 + lane;
      const int pg = idx / VCHUNKS, ch = idx - pg * VCHUNKS;
      const int pblk = __shfl(blk, pg * 16);
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (pblk >= 0)
        u = *reinterpret_cast<const uint4*>(a.cache + (int64_t)pblk * blk_stride + kvh * head_stride +
                                            a.f.vcodes + ch * 16);
      *reinterpret_cast<uint4*>(&vstage[wave][pg * 16 * VROW + ch * 16]) = u;
    }

    // Logits: rows = 4 query heads, columns = this lane's token, one coordinate per MFMA.
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kDim; ++i) {
      const uint32_t code = get_code<KB>(kw, i);
      acc = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[i], kcb[code], acc, 0, 0, 0);
    }
    floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QJL) {
#pragma unroll
      for (int i = 0; i < kDim; ++i) {
        const float sgn = ((sg[i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
        acc2 = __builtin_amdgcn_mfma_f32_4x4x1f32(p_lds[lane & 3][i], sgn, acc2, 0, 0, 0);
      }
    }
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
    // Online softmax (running max is wave-uniform; sums stay per lane).
    float wv[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float mnew = fmaxf(m_run[h], wave_max(lg[h]));
      float alpha = 1.f, pr = 0.f;
      if (mnew != -INFINITY) {
        alpha = __expf(m_run[h] - mnew);
        pr = valid ? __expf(lg[h] - mnew) : 0.f;
      }
      l_lane[h] = fmaf(l_lane[h], alpha, pr);
      if (!VLM) s_lane[h] = fmaf(s_lane[h], alpha, pr * va);
      O0[h] *= alpha;
      O1[h] *= alpha;
      m_run[h] = mnew;
      wv[h] = pr * (VLM ? va : vb);
    }
    wbuf[wave][lane] = make_float4(wv[0], wv[1], wv[2], wv[3]);
    wave_sync_lds();
    // Values: rows = 4 heads, columns = coordinates 2*lane / 2*lane+1, one token per MFMA.
    const uint8_t* vs = vstage[wave];
    const float* wb = reinterpret_cast<const float*>(wbuf[wave]);
#pragma unroll 8
    for (int tt = 0; tt < 64; ++tt) {
      const float wa = wb[4 * tt + (lane & 3)];
      const uint32_t pair = value_code_pair<VB>(vs + tt * VROW, lane);
      float b0, b1;
      if (VLM) {
        b0 = vcb[pair & ((1u << VB) - 1u)];
        b1 = vcb[pair >> VB];
      } else {
        b0 = (float)(pair & ((1u << VB) - 1u));
        b1 = (float)(pair >> VB);
      }
      O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(wa, b0, O0, 0, 0, 0);
      O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(wa, b1, O1, 0, 0, 0);
    }
    wave_sync_lds();
  }

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
    // to arrive merges all splits (log-sum-exp) and writes the output.
    if (h < G) {
      float* dst = a.ws + ((((int64_t)b * a.hkv + kvh) * a.splits + split) * 4 + h) * (2 + kDim);
      if (lane == 0) {
        dst[0] = M;
        dst[1] = L;
      }
      dst[2 + 2 * lane] = o0;
      dst[3 + 2 * lane] = o1;
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (tid == 0) {
      // wraps back to 0 after `splits` arrivals, so the counter is left zero
      const unsigned prev = __builtin_amdgcn_atomic_inc32(a.counters + (int64_t)b * a.hkv + kvh, (unsigned)(a.splits - 1),
                                                         __ATOMIC_ACQ_REL, "agent");
      last = prev == (unsigned)(a.splits - 1);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    M = -INFINITY;
    L = o0 = o1 = 0.f;
    if (h < G) {
      const int64_t stride = 4 * (2 + kDim);
      const float* src = a.ws + (((int64_t)b * a.hkv + kvh) * a.splits * 4 + h) * (2 + kDim);
      for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, src[sp * stride]);
      for (int sp = 0; sp < a.splits; ++sp) {
        const float ms = src[sp * stride];
        if (ms != -INFINITY) {
          const float f = __expf(ms - M);
          L = fmaf(f, src[sp * stride + 1], L);
          o0 = fmaf(f, src[sp * stride + 2 + 2 * lane], o0);
          o1 = fmaf(f, src[sp * stride + 3 + 2 * lane], o1);
        }
      }
    }
  }
  float r0 = L > 0.f ? o0 / L : 0.f;
  float r1 = L > 0.f ? o1 / L : 0.f;
  if constexpr (VLM) {
    // Lloyd-Max values were accumulated in the rotated basis: o = diag(s) H o' / sqrt(d).
    float* buf = &part_o[0][0][0] + h * kDim;      // reuse LDS: [4][128]
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
