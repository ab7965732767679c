// Quantize-append kernels for gfx950: stage-1 keys (random signs, in-register
// Walsh-Hadamard butterfly, Lloyd-Max codes through an LDS look-up grid, fp32
// norm with optional norm correction), optional QJL sign bits of S r computed
// on the fp32 matrix cores, and uniform or Lloyd-Max values.
//
// Sources (page and section): issoh.co.jp "TurboQuantとは？…", 第1段 and 第2段;
// lilting.ch TurboQuant article, QJL section and two-stage pipeline section
// (tokens are quantized once, online); ai-navigate-news turboquant-vllm write-up,
// "Bugs Nobody Else Has Found" (fp32 norms); qiita AMD LMCache article (two 4-bit
// codes per byte, low nibble first).
//
// One lane owns one (token, head) vector, so the 7-stage butterfly runs in that
// lane's registers without shuffles; for QJL keys each wave stages its 64
// residuals in LDS and multiplies them by S with 32x32x2 fp32 MFMA.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

// ---------------------------------------------------------------------------
// Keys.  Block of 256 lanes, one (token, head) vector per lane.
// ---------------------------------------------------------------------------
template <int KB, bool QJL, bool BF16>
__global__ __launch_bounds__(256) void append_keys_kernel(AppendArgs a) {
  __shared__ QLut lut[kLutCells];
  __shared__ float rbuf[QJL ? 4 : 1][QJL ? 64 : 1][QJL ? 33 : 1];
  __shared__ uint32_t sbits[QJL ? 4 : 1][QJL ? 64 : 1][4];
  for (int i = threadIdx.x; i < kLutCells; i += blockDim.x) lut[i] = a.c->klut[i];
  __syncthreads();

  const int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = th / a.hkv;
  const int h = (int)(th - t * a.hkv);
  int64_t slot = -1;
  if (t < a.num_tokens) slot = a.slots[t];
  const bool active = t < a.num_tokens && slot >= 0 && slot < a.num_blocks * kBlockTokensDev;
  if (!QJL && !active) return;

  uint32_t sb[4] = {a.sign_bits[0], a.sign_bits[1], a.sign_bits[2], a.sign_bits[3]};
  float x[kDim];
  if (active) {
    load_row<BF16>(a.k, th, x);
  } else {
#pragma unroll
    for (int i = 0; i < kDim; ++i) x[i] = 0.f;
  }
  uint32_t w[KB * 4];
  float cn2;
  float cres[QJL ? kDim : 1];
  const float n = lloyd_codes<KB, QJL>(x, sb, lut, a.klut_scale, a.klut_bias, w, cn2, cres);
  const float nhat = (a.key_nc && !QJL) ? n / sqrtf(cn2) : n;

  uint8_t* page = nullptr;
  int so = 0;
  if (active) {
    page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
    so = (int)(slot & 15);
    store_words<KB>(page + a.f.kcodes + so * (KB * 16), w);
    reinterpret_cast<float*>(page + a.f.knorm)[so] = nhat;
  }
  if constexpr (QJL) {
    // residual in the rotated frame: r'_i = H(s*k)_i / sqrt(d) - nhat * C[code_i]
    float r2 = 0.f;
#pragma unroll
    for (int i = 0; i < kDim; ++i) {
      x[i] = fmaf(-nhat, cres[i], x[i] * kInvSqrtDim);
      r2 = fmaf(x[i], x[i], r2);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    floatx16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][vt][r] = 0.f;
    // z[m][v] = sum_k S[m][k] r'_v[k] in four 32-coordinate chunks through LDS
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int j = 0; j < 32; ++j) rbuf[wave][lane][j] = x[32 * kc + j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int k = 32 * kc + 2 * kk + (lane >> 5);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          const float bv = rbuf[wave][32 * vt + (lane & 31)][2 * kk + (lane >> 5)];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const float av = a.c->St[k * kDim + 32 * mt + (lane & 31)];
            acc[mt][vt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[mt][vt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // sign bits: lane l holds column v = 32vt + l%32, rows 8(r/4) + 4(l/32) + r%4 of tile mt
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        uint32_t bits = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          bits |= (acc[mt][vt][r] >= 0.f ? 1u : 0u) << pos;
        }
        bits |= __shfl_xor(bits, 32);
        if (lane < 32) sbits[wave][32 * vt + lane][mt] = bits;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (active) {
      const uint4 sw = make_uint4(sbits[wave][lane][0], sbits[wave][lane][1], sbits[wave][lane][2],
                                  sbits[wave][lane][3]);
      reinterpret_cast<uint4*>(page + a.f.ksigns)[so] = sw;
      reinterpret_cast<float*>(page + a.f.kres)[so] = sqrtf(r2);
    }
  }
}

// ---------------------------------------------------------------------------
// Values.  Uniform: per-vector fp32 min and scale; Lloyd-Max: as plain keys.
// ---------------------------------------------------------------------------
template <int VB, bool VLM, bool BF16>
__global__ __launch_bounds__(256) void append_values_kernel(AppendArgs a) {
  __shared__ QLut lut[VLM ? kLutCells : 1];
  if (VLM) {
    for (int i = threadIdx.x; i < kLutCells; i += blockDim.x) lut[i] = a.c->vlut[i];
    __syncthreads();
  }
  const int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = th / a.hkv;
  if (t >= a.num_tokens) return;
  const int h = (int)(th - t * a.hkv);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * kBlockTokensDev) return;
  uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
  const int so = (int)(slot & 15);
  float x[kDim];
  load_row<BF16>(a.v, th, x);
  uint32_t w[VB * 4];
  if constexpr (VLM) {
    uint32_t sb[4] = {a.sign_bits[0], a.sign_bits[1], a.sign_bits[2], a.sign_bits[3]};
    float cn2;
    const float n = lloyd_codes<VB, false>(x, sb, lut, a.vlut_scale, a.vlut_bias, w, cn2, nullptr);
    reinterpret_cast<float*>(page + a.f.vmin)[so] = n;
  } else {
    float mn0 = x[0], mn1 = x[1], mx0 = x[0], mx1 = x[1];
#pragma unroll
    for (int i = 2; i < kDim; i += 2) {
      mn0 = fminf(mn0, x[i]); mx0 = fmaxf(mx0, x[i]);
      mn1 = fminf(mn1, x[i + 1]); mx1 = fmaxf(mx1, x[i + 1]);
    }
    const float mn = fminf(mn0, mn1), mx = fmaxf(mx0, mx1);
    constexpr float levels = (float)((1 << VB) - 1);
    const float sc = (mx - mn) / levels;               // correctly rounded division
    const float inv = sc > 0.f ? 1.f / sc : 0.f;
#pragma unroll
    for (int j = 0; j < VB * 4; ++j) w[j] = 0u;
#pragma unroll
    for (int i = 0; i < kDim; ++i) {
      // code = rint(fl32((x - mn) / sc)) with the correctly rounded fp32 quotient.  The
      // reciprocal product is within 2 ulp of it, so it decides the code unless it lies
      // within 2^-18 of a rounding boundary; only then take the exact division.
      const float d = x[i] - mn;
      float xq = d * inv;
      if (fabsf(xq - floorf(xq) - 0.5f) < 3.814697265625e-06f) xq = d / sc;
      const float q = fminf(rintf(xq), levels);                 // round half to even
      put_code<VB>(w, i, (uint32_t)q);
    }
    reinterpret_cast<float*>(page + a.f.vmin)[so] = mn;
    reinterpret_cast<float*>(page + a.f.vscale)[so] = sc;
  }
  store_planes<VB>(page + a.f.vcodes + so, w);
}

namespace {

inline unsigned blocks_for(int64_t threads, int per_block) {
  return (unsigned)((threads + per_block - 1) / per_block);
}

template <int KB, bool QJL>
hipError_t keys_for_dtype(const AppendArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(blocks_for(a.num_tokens * a.hkv, 256));
  if (dtype == TQ_BF16) hipLaunchKernelGGL((append_keys_kernel<KB, QJL, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_keys_kernel<KB, QJL, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int VB, bool VLM>
hipError_t values_for_dtype(const AppendArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(blocks_for(a.num_tokens * a.hkv, 256));
  if (dtype == TQ_BF16) hipLaunchKernelGGL((append_values_kernel<VB, VLM, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_values_kernel<VB, VLM, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB>
hipError_t keys_mode(const AppendArgs& a, int dtype, int key_mode, hipStream_t s) {
  return key_mode == TQ_KEY_LLOYD_QJL ? keys_for_dtype<KB, true>(a, dtype, s) : keys_for_dtype<KB, false>(a, dtype, s);
}

template <int VB>
hipError_t values_mode(const AppendArgs& a, int dtype, int val_mode, hipStream_t s) {
  return val_mode == TQ_VAL_LLOYD ? values_for_dtype<VB, true>(a, dtype, s) : values_for_dtype<VB, false>(a, dtype, s);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dtype, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s) {
  hipError_t e;
  switch (key_bits) {
    case 2: e = keys_mode<2>(a, dtype, key_mode, s); break;
    case 3: e = keys_mode<3>(a, dtype, key_mode, s); break;
    case 4: e = keys_mode<4>(a, dtype, key_mode, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (val_bits) {
    case 2: return values_mode<2>(a, dtype, val_mode, s);
    case 3: return values_mode<3>(a, dtype, val_mode, s);
    case 4: return values_mode<4>(a, dtype, val_mode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
