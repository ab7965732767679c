// PolarQuant keys for gfx950 (lilting.ch TurboQuant article, PolarQuant section:
// a vector's coordinate pairs become a radius and an angle, the radii are
// paired again down to one radius, and every angle is quantized on a uniform
// grid known in advance, so no per-block constants are stored).
//
// After the stage-1 rotation y = H(s*k)/sqrt(d), level 1 takes the angles of
// the 64 coordinate pairs (atan2, range [-pi, pi)), levels 2..7 the angles of
// pairs of radii (range [0, pi/2]); the last radius is ||k||, stored in fp32.
// Each angle gets a b-bit cell index; reconstruction uses the cell centre.  The
// 128 code slots are subtree-major: quarter g of the coordinates owns slots
// 32g..32g+31 (its 16 level-1, 8 level-2, 4 level-3, 2 level-4 and 1 level-5
// angles), and slot 32g+31 holds the root angle (g = 0), the level-6 angles
// (g = 1, 2) or padding (g = 3).  So the decode kernel's lane that holds
// coordinates 32g..32g+31 of a token also holds that quarter's codes.
//
// This file: the append kernel (one lane per token-head, the whole transform in
// registers) and the dequantize kernel (one lane per entry).  Decode lives in
// the decode kernel (key format kKmPolar).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_device.h"

namespace tq {

namespace {

__device__ __forceinline__ float wave_max_xor(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ double wave_sum64_xor(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------
// Append: keys only (the values go through the uniform values kernel).
// ---------------------------------------------------------------------------
template <int KB, bool BF16>
__global__ __launch_bounds__(256) void append_polar_kernel(AppendArgs a) {
  const int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = th / a.hkv;
  if (t >= a.num_tokens) return;
  const int h = (int)(th - t * a.hkv);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * kBlockTokensDev) return;
  float x[kDim];
  load_row<BF16>(a.k, th, x);
  const float radius = (float)sqrt(sumsq64(x));     // ||y|| = ||k||, fp64 sums rounded once
  uint32_t sb[4] = {a.sign_bits[0], a.sign_bits[1], a.sign_bits[2], a.sign_bits[3]};
  apply_signs(x, sb);
  wht128(x);
#pragma unroll
  for (int i = 0; i < kDim; ++i) x[i] *= kInvSqrtDim;
  uint32_t w[KB * 4];
#pragma unroll
  for (int j = 0; j < KB * 4; ++j) w[j] = 0u;
  // level by level: x[n] becomes the radius of node n
#pragma unroll
  for (int level = 1, n_nodes = kDim / 2; level <= 7; ++level, n_nodes >>= 1) {
#pragma unroll
    for (int n = 0; n < n_nodes; ++n) {
      const float u = x[2 * n], v = x[2 * n + 1];
      put_code<KB>(w, polar_slot(level, n), polar_code<KB>(atan2f(v, u), level == 1));
      x[n] = sqrtf(fmaf(u, u, v * v));
    }
  }
  uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
  const int so = (int)(slot & 15);
  store_words<KB>(page + a.f.kcodes + so * (KB * 16), w);
  reinterpret_cast<float*>(page + a.f.knorm)[so] = radius;
}

// ---------------------------------------------------------------------------
// Append of few rows (a decode step's new tokens): one wave per (token, head)
// row, keys and values together; lane l holds coordinates 2l and 2l+1 of both.
// The rotation is the butterfly across lanes.  Node n of tree level L sits in
// lane n 2^(L-1), its second child one exchange of 2^(L-2) lanes away.  Every
// value is computed with the same operations, in the same order, as in the
// one-lane-per-row kernels, so the bytes are the same.  Codes gather in LDS at
// their slots and leave as the packed row's bytes.  Values: the per-vector
// uniform rule (min, correctly rounded scale, codes) of the values kernel.
// ---------------------------------------------------------------------------
template <int KB, int VB, bool BF16>
__global__ __launch_bounds__(256) void append_polar_wave_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t kcod[4][kDim];
  __shared__ __align__(16) uint8_t vcod[4][kDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rows = a.num_tokens * a.hkv;
  const int64_t step = (int64_t)gridDim.x * 4;
  // sign word and bit of coordinates 2l, 2l+1
  const int sw = lane >> 4;
  const uint32_t sbits = sw == 0 ? a.sign_bits[0] : sw == 1 ? a.sign_bits[1] : sw == 2 ? a.sign_bits[2] : a.sign_bits[3];
  const uint32_t sg0 = ((sbits >> (2 * (lane & 15))) & 1u) << 31, sg1 = ((sbits >> (2 * (lane & 15) + 1)) & 1u) << 31;
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < rows; r += step) {   // uniform over the wave
    const int64_t t = r / a.hkv;
    const int h = (int)(r - t * a.hkv);
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_blocks * kBlockTokensDev) continue;
    uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
    const int so = (int)(slot & 15);
    float k0, k1, v0, v1;
    if constexpr (BF16) {
      const uint32_t kw = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k) + r * kDim)[lane];
      const uint32_t vw = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v) + r * kDim)[lane];
      k0 = bf16lo(kw); k1 = bf16hi(kw); v0 = bf16lo(vw); v1 = bf16hi(vw);
    } else {
      const float2 kk = reinterpret_cast<const float2*>(static_cast<const float*>(a.k) + r * kDim)[lane];
      const float2 vv = reinterpret_cast<const float2*>(static_cast<const float*>(a.v) + r * kDim)[lane];
      k0 = kk.x; k1 = kk.y; v0 = vv.x; v1 = vv.y;
    }
    // the stored radius ||y|| = ||k|| in fp64 from the inputs, rounded once
    const float radius = (float)sqrt(wave_sum64_xor(fma((double)k0, (double)k0, (double)k1 * (double)k1)));
    // keys: signs, the 128-point butterfly (coordinate bit 0 in the lane, bits
    // 1..6 across lanes 1..32 apart), 1/sqrt(d)
    k0 = __uint_as_float(__float_as_uint(k0) ^ sg0);
    k1 = __uint_as_float(__float_as_uint(k1) ^ sg1);
    float y0 = k0 + k1, y1 = k0 - k1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(y0, m), p1 = __shfl_xor(y1, m);
      const bool up = (lane & m) != 0;
      y0 = up ? p0 - y0 : y0 + p0;
      y1 = up ? p1 - y1 : y1 + p1;
    }
    y0 *= kInvSqrtDim;
    y1 *= kInvSqrtDim;
    if (lane == 0) kcod[wave][kDim - 1] = 0;                 // the unused slot
    kcod[wave][polar_slot(1, lane)] = (uint8_t)polar_code<KB>(atan2f(y1, y0), true);
    float rad = sqrtf(fmaf(y0, y0, y1 * y1));
#pragma unroll
    for (int lv = 2; lv <= 7; ++lv) {
      const float u = rad, v = __shfl_xor(rad, 1 << (lv - 2));
      if ((lane & ((1 << (lv - 1)) - 1)) == 0)
        kcod[wave][polar_slot(lv, lane >> (lv - 1))] = (uint8_t)polar_code<KB>(atan2f(v, u), false);
      rad = sqrtf(fmaf(u, u, v * v));
    }
    // values: per-vector min and correctly rounded scale
    const float mn = -wave_max_xor(-fminf(v0, v1));
    const float mx = wave_max_xor(fmaxf(v0, v1));
    constexpr float levels = (float)((1 << VB) - 1);
    const float sc = (mx - mn) / levels;
    const float inv = sc > 0.f ? 1.f / sc : 0.f;
    const float xv[2] = {v0, v1};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float d = xv[e] - mn;
      float xq = d * inv;
      if (fabsf(xq - floorf(xq) - 0.5f) < 3.814697265625e-06f) xq = d / sc;
      vcod[wave][2 * lane + e] = (uint8_t)fminf(rintf(xq), levels);
    }
    wave_sync_lds();
    if (lane < 16 * KB) page[a.f.kcodes + so * (KB * 16) + lane] = (uint8_t)stream_byte<KB>(kcod[wave], lane);
    if (lane < 16 * VB) page[a.f.vcodes + 16 * lane + so] = (uint8_t)stream_byte<VB>(vcod[wave], lane);
    if (lane == 0) {
      reinterpret_cast<float*>(page + a.f.knorm)[so] = radius;
      reinterpret_cast<float*>(page + a.f.vmin)[so] = mn;
      reinterpret_cast<float*>(page + a.f.vscale)[so] = sc;
    }
    wave_sync_lds();   // the codes are read before the next row overwrites them
  }
}

// ---------------------------------------------------------------------------
// Dequantize: one lane per (entry, head); k_hat = diag(s) H y_hat / sqrt(d),
// y_hat rebuilt top down from the radius and the cell-centre angles.
// ---------------------------------------------------------------------------
template <int KB, int VB, bool BF16OUT>
__global__ __launch_bounds__(128) void dequant_polar_kernel(DequantArgs a) {
  const int64_t th = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = th / a.hkv;
  if (i >= a.n) return;
  const int h = (int)(th - i * a.hkv);
  const int64_t rw = a.rows ? a.rows[i] : i;
  if (rw < 0 || rw >= a.buf_rows) return;
  const int64_t slot = a.slots[i];
  const bool ok = slot >= 0 && slot < a.num_blocks * kBlockTokensDev;
  float k[kDim], v[kDim];
#pragma unroll
  for (int c = 0; c < kDim; ++c) k[c] = v[c] = 0.f;
  if (ok) {
    const uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
    const int so = (int)(slot & 15);
    uint32_t w[KB * 4];
    const uint4* src = reinterpret_cast<const uint4*>(page + a.f.kcodes + so * (KB * 16));
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 u = src[j];
      w[4 * j] = u.x; w[4 * j + 1] = u.y; w[4 * j + 2] = u.z; w[4 * j + 3] = u.w;
    }
    // top down: k[n] holds the radius of node n of the current level
    k[0] = reinterpret_cast<const float*>(page + a.f.knorm)[so];
#pragma unroll
    for (int level = 7, n_nodes = 1; level >= 1; --level, n_nodes <<= 1) {
#pragma unroll
      for (int n = n_nodes - 1; n >= 0; --n) {
        const uint32_t code = get_code<KB>(w, polar_slot(level, n));
        const float* cs = level == 1 ? a.c->pcs1 : a.c->pcsU;
        const float r = k[n];
        k[2 * n] = r * cs[2 * code];
        k[2 * n + 1] = r * cs[2 * code + 1];
      }
    }
    uint32_t sb[4] = {a.sign_bits[0], a.sign_bits[1], a.sign_bits[2], a.sign_bits[3]};
    wht128(k);
#pragma unroll
    for (int c = 0; c < kDim; ++c) k[c] *= kInvSqrtDim;
    apply_signs(k, sb);
    uint32_t vw[VB * 4];
    load_planes<VB>(page + a.f.vcodes + so, vw);
    const float mn = reinterpret_cast<const float*>(page + a.f.vmin)[so];
    const float sc = reinterpret_cast<const float*>(page + a.f.vscale)[so];
#pragma unroll
    for (int c = 0; c < kDim; ++c) v[c] = fmaf(sc, (float)get_code<VB>(vw, c), mn);
  }
  const int64_t elem = (rw * a.hkv + h) * kDim;
  if constexpr (BF16OUT) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    uint32_t* ko = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.k_out) + elem);
    uint32_t* vo = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.v_out) + elem);
#pragma unroll
    for (int c = 0; c < kDim; c += 2) {
      ko[c / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){k[c], k[c + 1]}, bf16x2));
      vo[c / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v[c], v[c + 1]}, bf16x2));
    }
  } else {
    float4* ko = reinterpret_cast<float4*>(static_cast<float*>(a.k_out) + elem);
    float4* vo = reinterpret_cast<float4*>(static_cast<float*>(a.v_out) + elem);
#pragma unroll
    for (int c = 0; c < kDim; c += 4) {
      ko[c / 4] = make_float4(k[c], k[c + 1], k[c + 2], k[c + 3]);
      vo[c / 4] = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
    }
  }
}

namespace {

template <int KB>
hipError_t polar_keys(const AppendArgs& a, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)((a.num_tokens * a.hkv + 255) / 256));
  if (dtype == TQ_BF16) hipLaunchKernelGGL((append_polar_kernel<KB, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_polar_kernel<KB, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t polar_dequant(const DequantArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid((unsigned)((a.n * a.hkv + 127) / 128));
  if (bf16) hipLaunchKernelGGL((dequant_polar_kernel<KB, VB, true>), grid, dim3(128), 0, s, a);
  else hipLaunchKernelGGL((dequant_polar_kernel<KB, VB, false>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int KB>
hipError_t polar_dequant_vb(const DequantArgs& a, int val_bits, bool bf16, hipStream_t s) {
  switch (val_bits) {
    case 2: return polar_dequant<KB, 2>(a, bf16, s);
    case 3: return polar_dequant<KB, 3>(a, bf16, s);
    case 4: return polar_dequant<KB, 4>(a, bf16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_polar_keys(const AppendArgs& a, int dtype, int key_bits, hipStream_t s) {
  switch (key_bits) {
    case 2: return polar_keys<2>(a, dtype, s);
    case 3: return polar_keys<3>(a, dtype, s);
    case 4: return polar_keys<4>(a, dtype, s);
  }
  return hipErrorInvalidValue;
}

namespace {

template <int KB, int VB>
hipError_t polar_wave(const AppendArgs& a, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)std::min<int64_t>((a.num_tokens * a.hkv + 3) / 4, 8192));
  if (dtype == TQ_BF16) hipLaunchKernelGGL((append_polar_wave_kernel<KB, VB, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_polar_wave_kernel<KB, VB, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB>
hipError_t polar_wave_vb(const AppendArgs& a, int dtype, int val_bits, hipStream_t s) {
  switch (val_bits) {
    case 2: return polar_wave<KB, 2>(a, dtype, s);
    case 3: return polar_wave<KB, 3>(a, dtype, s);
    case 4: return polar_wave<KB, 4>(a, dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_polar_append_rows(const AppendArgs& a, int dtype, int key_bits, int val_bits, hipStream_t s) {
  switch (key_bits) {
    case 2: return polar_wave_vb<2>(a, dtype, val_bits, s);
    case 3: return polar_wave_vb<3>(a, dtype, val_bits, s);
    case 4: return polar_wave_vb<4>(a, dtype, val_bits, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_polar_dequant(const DequantArgs& a, int key_bits, int val_bits, bool bf16_out, hipStream_t s) {
  switch (key_bits) {
    case 2: return polar_dequant_vb<2>(a, val_bits, bf16_out, s);
    case 3: return polar_dequant_vb<3>(a, val_bits, bf16_out, s);
    case 4: return polar_dequant_vb<4>(a, val_bits, bf16_out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
