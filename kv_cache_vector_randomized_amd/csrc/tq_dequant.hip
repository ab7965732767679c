// Dequantize kernel for gfx950: stored codes back to fp32 vectors in the
// original basis (issoh.co.jp "TurboQuantとは？…", 第1段: the inverse of the
// random rotation is diag(s) H / sqrt(d); qiita AMD LMCache article: decoding is
// separate from byte transport, D(T(Q(X))) = D(Q(X))).
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

// ---------------------------------------------------------------------------
// Dequantize: one lane per (slot, head); keys k_hat = nhat * diag(s) H C[code] / sqrt(d).
// ---------------------------------------------------------------------------
template <int B, bool PLANES>
__device__ __forceinline__ void lloyd_decode_row(const uint8_t* row, float nrm, const float* cb,
                                                 const uint32_t (&sb)[4], float* out) {
  uint32_t w[B * 4];
  if constexpr (PLANES) {
    load_planes<B>(row, w);
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const uint4 u = src[j];
      w[4 * j] = u.x; w[4 * j + 1] = u.y; w[4 * j + 2] = u.z; w[4 * j + 3] = u.w;
    }
  }
  float x[kDim];
#pragma unroll
  for (int i = 0; i < kDim; ++i) x[i] = cb[get_code<B>(w, i)];
  wht128(x);
  const float f = nrm * kInvSqrtDim;
#pragma unroll
  for (int i = 0; i < kDim; ++i) x[i] *= f;
  apply_signs(x, sb);
  float4* o = reinterpret_cast<float4*>(out);
#pragma unroll
  for (int j = 0; j < 32; ++j) o[j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
}

template <int KB, int VB, bool VLM>
__global__ __launch_bounds__(128) void dequant_kernel(DequantArgs a) {
  __shared__ float kcb[16], vcb[16];
  if (threadIdx.x < 16) {
    kcb[threadIdx.x] = a.c->kc[threadIdx.x];
    vcb[threadIdx.x] = a.c->vc[threadIdx.x];
  }
  __syncthreads();
  const int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = th / a.hkv;
  if (i >= a.n) return;
  const int h = (int)(th - i * a.hkv);
  float* ko = a.k_out + th * kDim;
  float* vo = a.v_out + th * kDim;
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= a.num_blocks * kBlockTokensDev) {
    for (int j = 0; j < kDim; j += 4) {
      *reinterpret_cast<float4*>(ko + j) = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(vo + j) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
  const int so = (int)(slot & 15);
  uint32_t sb[4] = {a.sign_bits[0], a.sign_bits[1], a.sign_bits[2], a.sign_bits[3]};
  lloyd_decode_row<KB, false>(page + a.f.kcodes + so * (KB * 16), reinterpret_cast<const float*>(page + a.f.knorm)[so],
                       kcb, sb, ko);
  if constexpr (VLM) {
    lloyd_decode_row<VB, true>(page + a.f.vcodes + so, reinterpret_cast<const float*>(page + a.f.vmin)[so],
                         vcb, sb, vo);
  } else {
    uint32_t w[VB * 4];
    load_planes<VB>(page + a.f.vcodes + so, w);
    const float mn = reinterpret_cast<const float*>(page + a.f.vmin)[so];
    const float sc = reinterpret_cast<const float*>(page + a.f.vscale)[so];
#pragma unroll
    for (int j = 0; j < kDim; j += 4)
      *reinterpret_cast<float4*>(vo + j) =
          make_float4(fmaf(sc, (float)get_code<VB>(w, j), mn), fmaf(sc, (float)get_code<VB>(w, j + 1), mn),
                      fmaf(sc, (float)get_code<VB>(w, j + 2), mn), fmaf(sc, (float)get_code<VB>(w, j + 3), mn));
  }
}

namespace {

inline unsigned blocks_for(int64_t threads, int per_block) {
  return (unsigned)((threads + per_block - 1) / per_block);
}

template <int KB>
hipError_t dequant_vb(const DequantArgs& a, int val_bits, int val_mode, hipStream_t s) {
  const dim3 grid(blocks_for(a.n * a.hkv, 128));
  const bool lm = val_mode == TQ_VAL_LLOYD;
  switch (val_bits) {
    case 2:
      if (lm) hipLaunchKernelGGL((dequant_kernel<KB, 2, true>), grid, dim3(128), 0, s, a);
      else hipLaunchKernelGGL((dequant_kernel<KB, 2, false>), grid, dim3(128), 0, s, a);
      break;
    case 3:
      if (lm) hipLaunchKernelGGL((dequant_kernel<KB, 3, true>), grid, dim3(128), 0, s, a);
      else hipLaunchKernelGGL((dequant_kernel<KB, 3, false>), grid, dim3(128), 0, s, a);
      break;
    case 4:
      if (lm) hipLaunchKernelGGL((dequant_kernel<KB, 4, true>), grid, dim3(128), 0, s, a);
      else hipLaunchKernelGGL((dequant_kernel<KB, 4, false>), grid, dim3(128), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, int key_bits, int key_mode, int val_bits, int val_mode,
                          hipStream_t s) {
  (void)key_mode;
  switch (key_bits) {
    case 2: return dequant_vb<2>(a, val_bits, val_mode, s);
    case 3: return dequant_vb<3>(a, val_bits, val_mode, s);
    case 4: return dequant_vb<4>(a, val_bits, val_mode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
