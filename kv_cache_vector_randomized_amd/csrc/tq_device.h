// Device helpers shared by the HIP kernel files (rows, bit streams, the
// Hadamard butterfly, the code look-up grid).
#pragma once
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {


typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kInvSqrtDim = 0.08838834764831845f;   // 1/sqrt(128)

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One row of 128 activations (bf16 or fp32) into fp32 registers.
template <bool BF16>
__device__ __forceinline__ void load_row(const void* base, int64_t row, float (&x)[kDim]) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * kDim);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 w = p[j];
      x[8 * j + 0] = bf16lo(w.x); x[8 * j + 1] = bf16hi(w.x);
      x[8 * j + 2] = bf16lo(w.y); x[8 * j + 3] = bf16hi(w.y);
      x[8 * j + 4] = bf16lo(w.z); x[8 * j + 5] = bf16hi(w.z);
      x[8 * j + 6] = bf16lo(w.w); x[8 * j + 7] = bf16hi(w.w);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * kDim);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float4 w = p[j];
      x[4 * j + 0] = w.x; x[4 * j + 1] = w.y; x[4 * j + 2] = w.z; x[4 * j + 3] = w.w;
    }
  }
}

// In-place Sylvester (natural order) Walsh-Hadamard transform, unnormalized.
__device__ __forceinline__ void wht128(float (&x)[kDim]) {
#pragma unroll
  for (int len = 1; len < kDim; len <<= 1) {
#pragma unroll
    for (int i = 0; i < kDim; i += 2 * len) {
#pragma unroll
      for (int j = i; j < i + len; ++j) {
        const float a = x[j], b = x[j + len];
        x[j] = a + b;
        x[j + len] = a - b;
      }
    }
  }
}

__device__ __forceinline__ float sum_squares(const float (&x)[kDim]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int i = 0; i < kDim; i += 4) {
    s0 = fmaf(x[i], x[i], s0);
    s1 = fmaf(x[i + 1], x[i + 1], s1);
    s2 = fmaf(x[i + 2], x[i + 2], s2);
    s3 = fmaf(x[i + 3], x[i + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// Sum of squares accumulated in fp64: the square of an fp32 (or bf16) value is
// exact in fp64 and the sums keep 53 bits, so sqrt of the result rounded once to
// fp32 is within 1 ulp of the correctly rounded norm (stored norms are fp32 and
// must be accurate: ai-navigate-news turboquant-vllm write-up, "Bugs Nobody Else
// Has Found").
__device__ __forceinline__ double sumsq64(const float (&x)[kDim]) {
  double s0 = 0.0, s1 = 0.0;
#pragma unroll
  for (int i = 0; i < kDim; i += 2) {
    s0 = fma((double)x[i], (double)x[i], s0);
    s1 = fma((double)x[i + 1], (double)x[i + 1], s1);
  }
  return s0 + s1;
}

// code = #{j : t_j <= y} through the look-up grid; also returns C[code].
__device__ __forceinline__ int lut_code(const QLut* lut, float y, float sc, float bi, float& c) {
  const float f = fminf(fmaxf(fmaf(y, sc, bi), 0.f), (float)(kLutCells - 1));
  const QLut e = lut[(int)f];
  const bool up = y >= e.t;
  c = up ? e.c_hi : e.c_lo;
  return e.base + (up ? 1 : 0);
}

// 8-bit codes: code = #{j : t_j <= y} by binary search over the 255 ascending
// thresholds (each step keeps the count of thresholds known to be <= y); also
// returns C[code].
__device__ __forceinline__ int code_bsearch8(const float* t, const float* c, float y, float& cv) {
  int n = 0;
#pragma unroll
  for (int step = 128; step >= 1; step >>= 1)
    if (t[n + step - 1] <= y) n += step;
  cv = c[n];
  return n;
}

// Put code i (B bits) into an LSB-first bit stream held in 32-bit words.
template <int B>
__device__ __forceinline__ void put_code(uint32_t (&w)[B * 4], int i, uint32_t code) {
  const int bit = B * i, wi = bit >> 5, sh = bit & 31;
  w[wi] |= code << sh;
  if (sh + B > 32) w[wi + 1] |= code >> (32 - sh);
}

template <int B>
__device__ __forceinline__ uint32_t get_code(const uint32_t* w, int i) {
  const int bit = B * i, wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + B > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << B) - 1u);
}

template <int B>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t (&w)[B * 4]) {
  uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int j = 0; j < B; ++j) d[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
}

// Value codes are stored plane-major inside a page: byte p of the row of slot s
// sits at p * 16 + s (the 16 slots of one byte position are contiguous).
template <int B>
__device__ __forceinline__ void store_planes(uint8_t* dst_slot, const uint32_t (&w)[B * 4]) {
#pragma unroll
  for (int j = 0; j < B * 4; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) dst_slot[(4 * j + k) * 16] = (uint8_t)(w[j] >> (8 * k));
}

template <int B>
__device__ __forceinline__ void load_planes(const uint8_t* src_slot, uint32_t (&w)[B * 4]) {
#pragma unroll
  for (int j = 0; j < B * 4; ++j)
    w[j] = (uint32_t)src_slot[(4 * j) * 16] | ((uint32_t)src_slot[(4 * j + 1) * 16] << 8) |
           ((uint32_t)src_slot[(4 * j + 2) * 16] << 16) | ((uint32_t)src_slot[(4 * j + 3) * 16] << 24);
}

__device__ __forceinline__ void apply_signs(float (&x)[kDim], const uint32_t (&sb)[4]) {
#pragma unroll
  for (int i = 0; i < kDim; ++i)
    x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (((sb[i >> 5] >> (i & 31)) & 1u) << 31));
}

// Stage 1 on a vector already in registers: signs, norm, rotation, codes.
// On return x[i] holds the rotated, unnormalized coordinate H(s*x)_i and c[i]
// is not kept; returns ||x|| in fp64 and fills the packed words and sum C^2
// (fp64: the fp32 centroids' squares are exact there).
template <int B, bool KEEP_C>
__device__ __forceinline__ double lloyd_codes(float (&x)[kDim], const uint32_t (&sb)[4], const QLut* lut,
                                              float lsc, float lbi, uint32_t (&w)[B * 4], double& cn2,
                                              float* cvals, const float* t8 = nullptr, const float* c8 = nullptr) {
  const double n = sqrt(sumsq64(x));
  apply_signs(x, sb);
  const float n32 = sqrtf(sum_squares(x));   // scale of the code decisions only
  wht128(x);
  const float inv = n32 > 0.f ? 1.f / (n32 * 11.313708498984761f) : 0.f;
#pragma unroll
  for (int j = 0; j < B * 4; ++j) w[j] = 0u;
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int i = 0; i < kDim; ++i) {
    float c;
    const int code = B == 8 ? code_bsearch8(t8, c8, x[i] * inv, c) : lut_code(lut, x[i] * inv, lsc, lbi, c);
    put_code<B>(w, i, (uint32_t)code);
    if (i & 1) a1 = fma((double)c, (double)c, a1); else a0 = fma((double)c, (double)c, a0);
    if (KEEP_C) cvals[i] = c;
  }
  cn2 = a0 + a1;
  return n;
}

// Stored key norm: ||k|| (plain) or ||k|| / ||C[code]|| (corrected), from the
// fp64 sums, rounded once to fp32.  A zero key stores 0.
__device__ __forceinline__ float stored_norm(double n, double cn2, bool corrected) {
  return (float)(corrected ? (n > 0.0 ? n / sqrt(cn2) : 0.0) : n);
}
// The same from ||k||^2: sqrt(||k||^2 / ||C[code]||^2) (one fp64 square root).
__device__ __forceinline__ float stored_norm_sq(double n2, double cn2, bool corrected) {
  return (float)sqrt(corrected ? n2 / cn2 : n2);
}

// Make a wave's LDS writes visible to the wave's later LDS reads.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Byte p of the LSB-first bit stream of 128 codes of B bits held one per byte.
template <int B>
__device__ __forceinline__ uint32_t stream_byte(const uint8_t* codes, int p) {
  uint32_t v = 0u;
  for (int i = (8 * p) / B; i < kDim && B * i < 8 * p + 8; ++i) {
    const int sh = B * i - 8 * p;
    const uint32_t c = codes[i];
    v |= sh >= 0 ? (c << sh) : (c >> -sh);
  }
  return v & 0xFFu;
}

// E4M3 byte of x (FP8 keys): the nearest finite value with ties to the even
// code, magnitudes above 448 saturating to 448, the sign bit kept.  Every step is
// exact (power-of-two scalings, rint of an exactly scaled value).
__device__ __forceinline__ uint32_t fp8_e4m3(float x) {
  const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);   // subnormals: multiples of 2^-9 (8 = the smallest normal)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // floor(log2 a), -6..8
    const uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - e));           // 8..16; 16 carries
    code = (uint32_t)(8 * (e + 7)) + m - 8u;
  }
  return code | sgn;
}

// PolarQuant keys (lilting.ch TurboQuant article, PolarQuant section): slot of
// the angle of node `node` at tree level `level` in the 128-slot code row
// (subtree-major: quarter g of the coordinates owns slots 32g..32g+31; slot 31
// holds the root, slots 63 and 95 the two level-6 angles, slot 127 is unused),
// and the cell index of an angle: level 1 over [-pi, pi) (pi wraps to -pi),
// higher levels over [0, pi/2].
constexpr int polar_slot(int level, int node) {
  return level == 7 ? 31
       : level == 6 ? 32 * (node + 1) + 31
       : 32 * (node >> (5 - level)) +
             (level == 1 ? 0 : level == 2 ? 16 : level == 3 ? 24 : level == 4 ? 28 : 30) +
             (node & ((16 >> (level - 1)) - 1));
}

template <int B>
__device__ __forceinline__ uint32_t polar_code(float theta, bool level1) {
  constexpr float kPi = 3.14159265358979323846f;
  if (level1) {
    const float x = (theta + kPi) * ((float)(1 << B) / (2.f * kPi));
    return (uint32_t)(int)floorf(x) & ((1u << B) - 1u);
  }
  const float x = theta * ((float)(1 << B) / (0.5f * kPi));
  return (uint32_t)fminf(floorf(x), (float)((1 << B) - 1));
}

}  // namespace tq
