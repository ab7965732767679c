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
  constexpr bool WIDE = KB == 8;   // 8-bit codes: binary search over the thresholds instead of the grid
  __shared__ QLut lut[WIDE ? 1 : kLutCells];
  __shared__ float kt8[WIDE ? 256 : 1], kc8[WIDE ? 256 : 1];
  __shared__ float rbuf[QJL ? 4 : 1][QJL ? 64 : 1][QJL ? 33 : 1];
  __shared__ uint32_t sbits[QJL ? 4 : 1][QJL ? 64 : 1][4];
  if constexpr (WIDE) {
    kt8[threadIdx.x] = a.c->kt[threadIdx.x];   // blockDim.x == 256
    kc8[threadIdx.x] = a.c->kc[threadIdx.x];
  } else {
    for (int i = threadIdx.x; i < kLutCells; i += blockDim.x) lut[i] = a.c->klut[i];
  }
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
  double cn2;
  float cres[QJL ? kDim : 1];
  const double n = lloyd_codes<KB, QJL>(x, sb, lut, a.klut_scale, a.klut_bias, w, cn2, cres, kt8, kc8);
  const float nhat = stored_norm(n, cn2, a.key_nc && !QJL);

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
    double cn2;
    const double n = lloyd_codes<VB, false>(x, sb, lut, a.vlut_scale, a.vlut_bias, w, cn2, nullptr);
    reinterpret_cast<float*>(page + a.f.vmin)[so] = (float)n;
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

// ---------------------------------------------------------------------------
// FP8 keys with uniform values (issoh.co.jp "TurboQuantとは？…", preset table:
// keys in FP8, values in 4 bits).  A wave takes one (token, head) row at a time
// (rows handed out grid-stride); lane l holds coordinates 2l and 2l+1.  The key
// bytes form one 128-byte row; the values follow the per-vector kernel above
// (same min, scale and rounding), their codes gathered through LDS into the
// page's byte planes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_reduce_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

template <int VB, bool BF16>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t vcodes[4][kDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rows = a.num_tokens * a.hkv;
  const int64_t step = (int64_t)gridDim.x * 4;
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
    *reinterpret_cast<uint16_t*>(page + a.f.kcodes + so * kDim + 2 * lane) =
        (uint16_t)(fp8_e4m3(k0) | (fp8_e4m3(k1) << 8));
    const float mn = -wave_reduce_max(-fminf(v0, v1));
    const float mx = wave_reduce_max(fmaxf(v0, v1));
    constexpr float levels = (float)((1 << VB) - 1);
    const float sc = (mx - mn) / levels;               // correctly rounded division
    const float inv = sc > 0.f ? 1.f / sc : 0.f;
    float xv[2] = {v0, v1};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      // as the per-vector kernel: rint of the correctly rounded quotient, taken
      // exactly when the reciprocal product lies within 2^-18 of a boundary
      const float d = xv[e] - mn;
      float xq = d * inv;
      if (fabsf(xq - floorf(xq) - 0.5f) < 3.814697265625e-06f) xq = d / sc;
      vcodes[wave][2 * lane + e] = (uint8_t)fminf(rintf(xq), levels);
    }
    wave_sync_lds();
    if (lane < 16 * VB) page[a.f.vcodes + 16 * lane + so] = (uint8_t)stream_byte<VB>(vcodes[wave], lane);
    if (lane == 0) {
      reinterpret_cast<float*>(page + a.f.vmin)[so] = mn;
      reinterpret_cast<float*>(page + a.f.vscale)[so] = sc;
    }
    wave_sync_lds();   // the codes are read before the next row overwrites them
  }
}

// ---------------------------------------------------------------------------
// Keys and values of whole pages, bf16 inputs (Lloyd-Max keys without QJL,
// uniform values).  A work-group of 4 waves takes pairs of groups of 16
// consecutive tokens of one KV head: two waves quantize the keys of the two
// groups, the other two their values, the roles swapping from pass to pass.
// When a group's slots are the 16 slots of one page in order (prefill), the
// page's value planes are assembled in LDS and written with one 16-byte store
// per plane; otherwise every token goes to its own slot.
//
// Rotation on the matrix cores.  Write a coordinate as 7 bits c = (c6..c0); the
// Sylvester matrix is the product over bits of (-1)^(out_b * in_b), so it
// factors over any split of the bits.  The bf16 MFMA (16x16x16, fp32 sums)
// applies the 16-point transform over bits {0, 1, 3, 4} with the sign-flipped
// rows as its B operand (exact bf16 values); the 8-point transform over bits
// {2, 5, 6} is a 24-add butterfly inside each lane.  Lane (j, g) = (lane % 16,
// lane / 16) loads 16-byte chunks g, g+4, g+8, g+12 of token j's row and ends
// with rotated coordinates 32n + 8g + (0..7), n = 0..3, of token j: 8
// consecutive codes per n, i.e. whole packed bytes.
//
// Codes: g = 128 y; the fp32 sum g + (1.5 * 2^23 + 128) carries the grid cell
// round(g) + 128 in its low mantissa bits, and shifting its bit pattern left by
// 4 and adding a constant gives the LDS address of the cell (mod 2^32).
// ---------------------------------------------------------------------------
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr float kUnitMagic = 12583040.0f;     // 1.5 * 2^23 + 128; bit pattern 0x4B400080

// min over the 4 lanes of each quad for `mn`, max for `mx` (every lane gets
// them).  The s_nop instructions cover the DPP read-after-VALU-write hazard.
__device__ __forceinline__ void quad_minmax(float& mn, float& mx) {
  asm volatile(
      "s_nop 1\n\t"
      "v_min_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_min_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "+v"(mn), "+v"(mx));
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 mfma_f16x32(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0,
                                                0);
}

// Sum over the lanes j, j+16, j+32, j+48.
__device__ __forceinline__ float sum_rows(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}
__device__ __forceinline__ double sum_rows64(double v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

template <int KB, int VB, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QJL ? 2 : 3))) void append_page_kernel(AppendArgs a) {
  constexpr int KROW = 16 * KB;            // bytes of a packed key row
  constexpr int VROW = 16 * VB;            // bytes of a packed value row (= planes)
  constexpr int KSTR = KROW + 16;          // LDS stride of a packed key row
  __shared__ __align__(16) QLut lut[kUnitCellsPadded];
  __shared__ __align__(16) uint8_t kpack[4][16][KSTR];    // packed key rows [wave][token]
  __shared__ __align__(16) uint8_t vplane[4][64][16];     // value planes [wave][plane][token]
  // ||k||^2 (fp64) of the wave's 16 tokens, parked in LDS across the code loop
  // (volatile: kept out of registers, where it would push the kernel into spills)
  __shared__ volatile double knorm_lds[4][16];
  // sum of C[code]^2 (fp64, the fp32 centroids' squares exact) of every field of a packed
  // key row: a byte of 4-bit or 2-bit codes, 6 bits (two codes) of 3-bit codes
  constexpr int kFieldBits = KB == 3 ? 6 : 8;
  __shared__ double c2tab[QJL ? 1 : 1 << kFieldBits];
  // QJL: the f16 terms of S in the operand order of the MFMA (see the key pass)
  __shared__ __align__(16) uint32_t sq[QJL ? kDim * kDim : 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = wave & 1;                 // which group of the pair
  // (the launcher keeps the group count below 2^31)
  const uint32_t hkv = (uint32_t)a.hkv;
  const uint32_t ngroups = (uint32_t)((a.num_tokens + 15) / 16) * hkv;
  const uint32_t npairs = (ngroups + 1) / 2;
  const int64_t tmax = a.num_tokens - 1;

  // Group 2p + wg of the pair p: its first token and head; a group past the end
  // (odd count) stands in for the last one and writes nothing.
  auto group_of = [&](uint32_t p, int64_t& t0, int& h) -> bool {
    const uint32_t grp = 2u * p + (uint32_t)wg;
    const bool live = grp < ngroups;
    const uint32_t gg = live ? grp : ngroups - 1;
    const uint32_t tb = gg / hkv;
    h = (int)(gg - tb * hkv);
    t0 = (int64_t)tb * 16;
    return live;
  };
  // Inputs and raw slot of this lane's token; loads are unconditional (indices
  // clamped), and nothing here waits for them.
  // Keys: lane (j, g) = (lane % 16, lane / 16) reads chunks g + 4n of token j.
  // Values: lane (t, q) = (lane / 4, lane % 4) reads chunks q + 4n of token t.
  auto load_group = [&](uint32_t p, bool keys, uint4 (&dst)[4], int64_t& raw) {
    int64_t t0;
    int h;
    (void)group_of(p, t0, h);
    const int tok = keys ? (lane & 15) : (lane >> 2);
    const int cg = keys ? (lane >> 4) : (lane & 3);
    const int64_t t = min(t0 + tok, tmax);
    const uint16_t* src = static_cast<const uint16_t*>(keys ? a.k : a.v) + (t * a.hkv + h) * kDim + 8 * cg;
#pragma unroll
    for (int n = 0; n < 4; ++n) dst[n] = *reinterpret_cast<const uint4*>(src + 32 * n);
    raw = a.slots[t];
  };

  // In pass i the waves 0, 1 (i even) or 2, 3 (i odd) quantize the keys of the
  // pair's two groups and the other two their values, so that every SIMD gets
  // both kinds of work.
  // Pair of round r for this work-group (npairs: none), per the launcher's round plan;
  // round 0 is pair blockIdx.x (the launcher keeps gridDim.x <= npairs).
  const uint32_t slot_wgs = (uint32_t)a.slot_wgs;
  const uint32_t my_rounds = (uint32_t)a.rounds[min(blockIdx.x / slot_wgs, 2u)];
  auto pair_of = [&](uint32_t r) -> uint32_t {
    if (r >= my_rounds) return npairs;
    const uint32_t q = slot_wgs * (min(r, (uint32_t)a.rounds[0]) + min(r, (uint32_t)a.rounds[1]) +
                                   min(r, (uint32_t)a.rounds[2])) + blockIdx.x;
    return q < npairs ? q : npairs;
  };
  uint32_t p = blockIdx.x;
  uint32_t round = 0;
  const bool keys0 = wave < 2;             // role in even passes
  uint4 inA[4], inB[4];
  int64_t rawA, rawB;
  load_group(p, keys0, inA, rawA);
  for (int i = threadIdx.x; i < kUnitCellsPadded; i += 256)
    *reinterpret_cast<uint4*>(&lut[i]) = *reinterpret_cast<const uint4*>(&a.c->kulut[i]);
  if constexpr (QJL) {
    for (int i = threadIdx.x; i < kDim * kDim / 4; i += 256)
      *reinterpret_cast<uint4*>(&sq[4 * i]) = *reinterpret_cast<const uint4*>(&a.c->Sh[4 * i]);
  } else {
    for (int i = threadIdx.x; i < (1 << kFieldBits); i += 256) {
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < kFieldBits / KB; ++q) {
        const double c = (double)a.c->kc[(i >> (KB * q)) & ((1 << KB) - 1)];
        t = fma(c, c, t);
      }
      c2tab[i] = t;
    }
  }
  // A operands of the key rotation, one per block b = beta + 2n of the 16-point
  // transform: H16[j][k] times the sign of coordinate 32n + 8(k/4) + 4beta + k%4
  // (k = 4g + e), so the bf16 rows enter the MFMA as they are.
  shortx4 hs[8];
  {
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = 8 * g + 4 * (b & 1) + e;
        const uint32_t neg = ((a.sign_bits[b >> 1] >> bit) ^ (uint32_t)__builtin_popcount(j & (4 * g + e))) & 1u;
        hs[b][e] = (short)(0x3F80u | (neg << 15));
      }
  }
  __syncthreads();

  // One pass: pair p's group wg, keys or values, from inputs `in` and raw slot
  // `raw` (loaded one pass earlier).
  auto run_pass = [&](uint32_t p, bool keys, const uint4 (&in)[4], int64_t raw) {
      int64_t t0;
      int h;
      const bool live = group_of(p, t0, h);
      // this lane's slot, -1 when its token or slot is out of range (or the group is)
      const int64_t slot = (live && t0 + (keys ? (lane & 15) : (lane >> 2)) <= tmax && raw >= 0 &&
                            raw < a.num_blocks * kBlockTokensDev) ? raw : -1;
      auto page_of = [&](int64_t s) -> uint8_t* { return a.cache + ((s >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes; };

      if (keys) {
        const int j = lane & 15, g = lane >> 4;
        // z[b], b = beta + 2n: the 16-point transform of the signed coordinates
        // 32n + 8g' + 4beta + e
        floatx4 z[8];
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          z[2 * n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              hs[2 * n], __builtin_bit_cast(shortx4, make_uint2(in[n].x, in[n].y)), zero, 0, 0, 0);
          z[2 * n + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              hs[2 * n + 1], __builtin_bit_cast(shortx4, make_uint2(in[n].z, in[n].w)), zero, 0, 0, 0);
        }
        // ||k|| of the stored norm from the bf16 inputs in fp64 (squares exact), while
        // the rotation runs on the matrix cores
        double kk0 = 0.0, kk1 = 0.0;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const uint32_t wv[4] = {in[n].x, in[n].y, in[n].z, in[n].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kk0 = fma((double)bf16lo(wv[e]), (double)bf16lo(wv[e]), kk0);
            kk1 = fma((double)bf16hi(wv[e]), (double)bf16hi(wv[e]), kk1);
          }
        }
        const double kkt = sum_rows64(kk0 + kk1);
        // QJL keys store the plain norm, known now; the corrected norm waits for the codes
        if constexpr (QJL) {
          if (g == 0 && slot >= 0) reinterpret_cast<float*>(page_of(slot) + a.f.knorm)[slot & 15] = (float)sqrt(kkt);
        } else {
          if (g == 0) knorm_lds[wave][j] = kkt;
        }
        // QJL: the residual in the rotated frame, times sqrt(d): z - sqrt(d) ||k|| C[code]
        const float nz = QJL ? (float)sqrt(128.0 * kkt) : 0.f;
        __builtin_amdgcn_sched_barrier(0);     // keep the fp64 sums' registers out of the code loop
        // 8-point butterfly over b: z[b][r] becomes coordinate 32(b/2) + 8g + 4(b%2) + r
#pragma unroll
        for (int len = 1; len < 8; len <<= 1)
#pragma unroll
          for (int i = 0; i < 8; i += 2 * len)
#pragma unroll
            for (int m = i; m < i + len; ++m) {
              const floatx4 u = z[m], v = z[m + len];
              z[m] = u + v;
              z[m + len] = u - v;
            }
        // u = y / ||y||, g = 128 u = sqrt(d) z / ||k|| (||z|| = sqrt(d) ||k||); a zero key gives
        // g = 0, codes 2^(b-1) and norm 0
        const float kkf = (float)kkt;
        const float sg = kkf > 0.f ? 11.313708498984761f * __builtin_amdgcn_rsqf(kkf) : 0.f;
        const uint32_t lut_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) QLut*)lut + 0x4C000000u;
        double c2 = 0.0;
        uint32_t w[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          uint32_t wn = 0u;
          if constexpr (QJL) {
            // two cells requested at a time (16-byte reads: the centroids come along);
            // one at a time waits out every LDS round trip at two waves per SIMD
#pragma unroll
            for (int pr2 = 0; pr2 < 4; ++pr2) {
              floatx4& zz = z[2 * n + (pr2 >> 1)];
              float gv[2];
              u32x4 e[2];
#pragma unroll
              for (int r = 0; r < 2; ++r) {
                gv[r] = zz[2 * (pr2 & 1) + r] * sg;
                const uint32_t addr = (__float_as_uint(gv[r] + kUnitMagic) << 4) + lut_addr;
                e[r] = *reinterpret_cast<lds_u32x4*>((uintptr_t)addr);
              }
#pragma unroll
              for (int r = 0; r < 2; ++r) {
                const bool up = gv[r] >= __uint_as_float(e[r].y);
                const float c = up ? __uint_as_float(e[r].w) : __uint_as_float(e[r].z);
                zz[2 * (pr2 & 1) + r] = fmaf(-nz, c, zz[2 * (pr2 & 1) + r]);
                wn |= (e[r].x + (uint32_t)up) << (KB * (2 * pr2 + r));
              }
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float gv = z[2 * n + (i >> 2)][i & 3] * sg;
              const uint32_t addr = (__float_as_uint(gv + kUnitMagic) << 4) + lut_addr;
              const u32x4 e = *reinterpret_cast<lds_u32x4*>((uintptr_t)addr);
              wn |= (e.x + (uint32_t)(gv >= __uint_as_float(e.y))) << (KB * i);
            }
          }
          w[n] = wn;
        }
        if constexpr (!QJL) {
          // ||C[code]||^2 of the corrected norm from the packed codes, field by field
          if (a.key_nc) {
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int f = 0; f < 8 * KB / kFieldBits; ++f)
                c2 += c2tab[(w[n] >> (kFieldBits * f)) & ((1u << kFieldBits) - 1)];
            c2 = sum_rows64(c2);
          }
        }
        if (!QJL && g == 0 && slot >= 0)
          reinterpret_cast<float*>(page_of(slot) + a.f.knorm)[slot & 15] =
              stored_norm_sq(knorm_lds[wave][j], c2, a.key_nc);
        if constexpr (QJL) {
          // p = S r~ on the f16 16x16x32 MFMA, each side split into two f16 terms
          // (r~ scaled by a power of two per token: signs do not change):
          // p = S_hi r_hi + S_hi r_lo + S_lo r_hi, the dropped S_lo r_lo and the
          // terms' own rounding below 2^-22 |S_i| |r~| each (Cauchy-Schwarz), far
          // inside the 1e-6 band of the sign decision.  Rows = 16 rows of S (tile
          // mt), columns = the 16 tokens, K step n = coordinates 32n + 8g + e of
          // lane (j, g): the lane's own registers are its B operand.
          float rr = 0.f;
#pragma unroll
          for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) rr = fmaf(z[b][r], z[b][r], rr);
          rr = sum_rows(rr);
          // |r~_i| <= ||z|| (1 + max |C|) < 2^(e+1) with ||z|| in [2^(e-1), 2^e)
          const float rs = ldexpf(1.f, 13 - __builtin_amdgcn_frexp_expf(nz));
          uint4 rh[4], rl[4];
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int p2 = 0; p2 < 4; ++p2) {
              const float v0 = z[2 * n + (p2 >> 1)][2 * (p2 & 1)] * rs;
              const float v1 = z[2 * n + (p2 >> 1)][2 * (p2 & 1) + 1] * rs;
              const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
              const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
              hw[p2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
              lw[p2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
            }
            rh[n] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            rl[n] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
          }
          // Sign rows of the wave's 16 tokens: lane (j, g) computes bits 16mt + 4g + r
          // (mt = 0..7, r = 0..3) of token j's row, nibble mt of `mine`.
          // p >= 0 is read off the fp32 sign bit: the accumulators start at +0 and add
          // finite terms, so p is never -0 or NaN.  Each step shifts `neg` left by one
          // and brings in the sign bit of p (one funnel shift), so the bit of step
          // k = 4mt + r ends at 31 - k; one bit reversal and a complement give `mine`.
          uint32_t neg = 0u;
#pragma unroll 2
          for (int mt = 0; mt < 8; ++mt) {
            // the three products in separate accumulators: three MFMA chains instead of one
            floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc, acc2 = acc;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              const uint4 sh = *reinterpret_cast<const uint4*>(&sq[(((0 * 8 + mt) * 4 + n) * 64 + lane) * 4]);
              const uint4 sl = *reinterpret_cast<const uint4*>(&sq[(((1 * 8 + mt) * 4 + n) * 64 + lane) * 4]);
              acc1 = mfma_f16x32(sl, rh[n], acc1);
              acc2 = mfma_f16x32(sh, rl[n], acc2);
              acc = mfma_f16x32(sh, rh[n], acc);
            }
            acc = acc + (acc1 + acc2);
            // lane (j, g) holds p[16mt + 4g + r] of token j
#pragma unroll
            for (int r = 0; r < 4; ++r) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(acc[r]), 31);
          }
          const uint32_t mine = __builtin_bitreverse32(~neg);
          // Dword g of token j's row (rows 32g..32g+31) takes nibbles 2g and 2g+1
          // of each lane (j, g'), at bits 4g' + r and 16 + 4g' + r.
          uint32_t srw = 0u;
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const uint32_t byte = ((uint32_t)__shfl((int)mine, j + 16 * gg) >> (8 * g)) & 0xFFu;
            srw |= ((byte & 0xFu) << (4 * gg)) | ((byte >> 4) << (16 + 4 * gg));
          }
          if (slot >= 0) {
            uint8_t* pg = page_of(slot);
            // lane g stores dword g of token j's sign row
            reinterpret_cast<uint32_t*>(pg + a.f.ksigns + 16 * (slot & 15))[g] = srw;
            if (g == 0) reinterpret_cast<float*>(pg + a.f.kres)[slot & 15] = sqrtf(rr) * kInvSqrtDim;
          }
        }
        // codes of coordinates 32n + 8g .. +7 are bytes KB*(4n + g) .. +KB-1 of the row
        uint8_t* prow = &kpack[wave][j][0];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int o = KB * (4 * n + g);
          if constexpr (KB == 4) *reinterpret_cast<uint32_t*>(prow + o) = w[n];
          else if constexpr (KB == 2) *reinterpret_cast<uint16_t*>(prow + o) = (uint16_t)w[n];
          else {
            prow[o] = (uint8_t)w[n];
            prow[o + 1] = (uint8_t)(w[n] >> 8);
            prow[o + 2] = (uint8_t)(w[n] >> 16);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Key rows: lane l stores bytes 4*KB*(l%4) .. +4*KB-1 of token l/4's row.
        const int kv = lane >> 2, kq = lane & 3;
        const int64_t slot_kv = __builtin_amdgcn_ds_bpermute(kv << 2, (int)slot) |
                                ((int64_t)__builtin_amdgcn_ds_bpermute(kv << 2, (int)(slot >> 32)) << 32);
        if (slot_kv >= 0) {
          const uint8_t* srow = &kpack[wave][kv][4 * KB * kq];
          uint8_t* dst = page_of(slot_kv) + a.f.kcodes + (slot_kv & 15) * KROW + 4 * KB * kq;
          if constexpr (KB == 4) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(srow);
          else if constexpr (KB == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(srow);
          else {
            const uint32_t* s32 = reinterpret_cast<const uint32_t*>(srow);
            uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
            d32[0] = s32[0]; d32[1] = s32[1]; d32[2] = s32[2];
          }
        }
      } else {
        const int t = lane >> 2, q = lane & 3;
        const int64_t slot0 = __builtin_amdgcn_readfirstlane((int)slot) |
                              ((int64_t)__builtin_amdgcn_readfirstlane((int)(slot >> 32)) << 32);
        // the 16 tokens fill one page in order
        const bool whole = (__ballot(!(slot >= 0 && slot == slot0 + t)) == 0ull) && slot0 >= 0 && (slot0 & 15) == 0;

        float x[32];                              // x[8n + e]: coordinate 32n + 8q + e
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const uint32_t wv[4] = {in[n].x, in[n].y, in[n].z, in[n].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            x[8 * n + 2 * d] = bf16lo(wv[d]);
            x[8 * n + 2 * d + 1] = bf16hi(wv[d]);
          }
        }
        float mn = x[0], mx = x[0];
#pragma unroll
        for (int k = 1; k < 32; ++k) {
          mn = fminf(mn, x[k]);
          mx = fmaxf(mx, x[k]);
        }
        quad_minmax(mn, mx);
        constexpr float levels = (float)((1 << VB) - 1);
        const float sc = (mx - mn) / levels;                  // correctly rounded division
        const float inv = sc > 0.f ? 1.f / sc : 0.f;          // correctly rounded
        // code = rint(fl32(x - mn) * inv), round half to even.  The product is within 2 ulp
        // of the exact quotient (x - mn) / sc, so it decides as the exact quotient does
        // unless that lies within about 2^-20 of a rounding boundary: a normalised distance
        // (x - mn) / (mx - mn) far below 1e-6, inside the band where either code counts.
        // v_cvt_pk_u8_f32 rounds to nearest even and writes the code into one byte of a
        // word; codes e and e + 4 share a word, and the words of 4-bit (2-bit) codes merge
        // with one shift-or (three) into the packed stream.
        uint32_t w[4];                            // w[n]: the 8 codes of chunk q + 4n (VB bytes)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const float* xn = &x[8 * n];
          if constexpr (VB == 4 || VB == 2) {
            uint32_t by[4];                       // by[r]: byte k = code r + 4k (VB 4: r + 2k)
            constexpr int per = 8 / VB;           // codes per byte
#pragma unroll
            for (int r = 0; r < per; ++r) {
              uint32_t t = 0u;
#pragma unroll
              for (int k = 0; k < VB; ++k) t = __builtin_amdgcn_cvt_pk_u8_f32((xn[r + per * k] - mn) * inv, k, t);
              by[r] = t;
            }
            uint32_t wn = by[0];
#pragma unroll
            for (int r = 1; r < per; ++r) wn |= by[r] << (VB * r);
            w[n] = wn;
          } else {
            uint32_t wn = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) wn |= (uint32_t)rintf((xn[e] - mn) * inv) << (VB * e);
            w[n] = wn;
          }
        }
        if (q == 0 && slot >= 0) {
          uint8_t* pg = page_of(slot);
          reinterpret_cast<float*>(pg + a.f.vmin)[slot & 15] = mn;
          reinterpret_cast<float*>(pg + a.f.vscale)[slot & 15] = sc;
        }
        // row bytes VB*(q + 4n) .. +VB-1 are those planes
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int i = 0; i < VB; ++i) vplane[wave][VB * (q + 4 * n) + i][t] = (uint8_t)(w[n] >> (8 * i));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Value planes: a whole page takes one 16-byte store per plane; otherwise
        // each token's byte of each plane goes to its own slot.
        if (whole) {
          if (lane < VROW)
            *reinterpret_cast<uint4*>(page_of(slot0) + a.f.vcodes + 16 * lane) =
                *reinterpret_cast<const uint4*>(&vplane[wave][lane][0]);
        } else {
#pragma unroll 1
          for (int v = 0; v < 16; ++v) {
            const int64_t sv = __builtin_amdgcn_readlane((int)slot, 4 * v) |
                               ((int64_t)__builtin_amdgcn_readlane((int)(slot >> 32), 4 * v) << 32);
            if (sv >= 0 && lane < VROW) page_of(sv)[a.f.vcodes + 16 * lane + (sv & 15)] = vplane[wave][lane][v];
          }
        }
      }
    // the LDS rows of this wave are rewritten next pass: keep this pass's reads first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Pairs of rounds 0, 1, ...: the next pair's inputs are loaded while this one
  // is quantized, into the other of two register sets (a copy of registers still
  // being loaded would wait for the load).
  for (;;) {
    uint32_t pn = pair_of(++round);
    bool more = pn < npairs;
    load_group(more ? pn : p, !keys0, inB, rawB);
    run_pass(p, keys0, inA, rawA);
    if (!more) break;
    p = pn;
    pn = pair_of(++round);
    more = pn < npairs;
    load_group(more ? pn : p, keys0, inA, rawA);
    run_pass(p, !keys0, inB, rawB);
    if (!more) break;
    p = pn;
  }
}

namespace {
template <bool QJL>
const void* page_ptr(int key_bits, int val_bits) {
  switch (key_bits * 8 + val_bits) {
    case 2 * 8 + 2: return (const void*)append_page_kernel<2, 2, QJL>;
    case 2 * 8 + 3: return (const void*)append_page_kernel<2, 3, QJL>;
    case 2 * 8 + 4: return (const void*)append_page_kernel<2, 4, QJL>;
    case 3 * 8 + 2: return (const void*)append_page_kernel<3, 2, QJL>;
    case 3 * 8 + 3: return (const void*)append_page_kernel<3, 3, QJL>;
    case 3 * 8 + 4: return (const void*)append_page_kernel<3, 4, QJL>;
    case 4 * 8 + 2: return (const void*)append_page_kernel<4, 2, QJL>;
    case 4 * 8 + 3: return (const void*)append_page_kernel<4, 3, QJL>;
    case 4 * 8 + 4: return (const void*)append_page_kernel<4, 4, QJL>;
  }
  return nullptr;
}
}  // namespace

const void* append_page_kernel_ptr(int key_bits, int val_bits, bool qjl) {
  return qjl ? page_ptr<true>(key_bits, val_bits) : page_ptr<false>(key_bits, val_bits);
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

template <int KB, bool QJL>
hipError_t page_vb(const AppendArgs& args, int val_bits, hipStream_t s) {
  // one pair of 16-token groups per work-group and pass; at most a.page_wgs work-groups
  AppendArgs a = args;
  const int64_t pairs = ((a.num_tokens + 15) / 16 * a.hkv + 1) / 2;
  const int64_t wgs = std::max(1, a.page_wgs);
  const dim3 grid((unsigned)std::min<int64_t>(pairs, wgs));
  // Round plan.  The resident work-groups of a compute unit do not progress at the
  // same rate: the first dispatched to it (ids below wgs / n with n per unit, as
  // the dispatcher fills every unit once before the next) issue first and finish
  // earlier.  Long appends give the slots of each unit shares of its pairs that
  // make them end together: 120 : 110 : 100 with three work-groups per unit
  // (1.7% faster than equal shares on 131072 tokens x 8 heads), 130 : 100 with
  // two (the QJL kernel: about 2.5% faster on 8 x 16384 tokens x 8 heads), the
  // best of the shares timed.  Other appends take pairs round-robin (one slot).  Every
  // pair belongs to exactly one (work-group, round) either way; the plan only
  // moves work, never drops it.
  a.slot_wgs = (int32_t)grid.x;
  a.rounds[0] = (int32_t)((pairs + grid.x - 1) / grid.x);
  a.rounds[1] = a.rounds[2] = 0;
  const int ns = a.page_per_cu;
  if ((ns == 2 || ns == 3) && (int64_t)grid.x == wgs && wgs % ns == 0 && pairs >= 8 * wgs) {
    const int64_t c = wgs / ns;
    const int64_t per_unit = (pairs + c - 1) / c;
    const int64_t w[3] = {ns == 3 ? 120 : 130, ns == 3 ? 110 : 100, ns == 3 ? 100 : 0};
    const int64_t wsum = w[0] + w[1] + w[2];
    int64_t n[3] = {0, 0, 0}, sum = 0;
    for (int i = 0; i < ns; ++i) {
      n[i] = per_unit * w[i] / wsum;
      sum += n[i];
    }
    for (int i = 0; sum < per_unit; i = (i + 1) % ns, ++sum) ++n[i];   // the remainder to the first slots
    a.slot_wgs = (int32_t)c;
    for (int i = 0; i < 3; ++i) a.rounds[i] = (int32_t)n[i];
  }
  switch (val_bits) {
    case 2: hipLaunchKernelGGL((append_page_kernel<KB, 2, QJL>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((append_page_kernel<KB, 3, QJL>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((append_page_kernel<KB, 4, QJL>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dtype, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s) {
  if (key_mode == TQ_KEY_POLAR) {
    if (val_mode != TQ_VAL_UNIFORM) return hipErrorInvalidValue;
    if (a.num_tokens * a.hkv <= kPolarWaveRows) return launch_polar_append_rows(a, dtype, key_bits, val_bits, s);
    const hipError_t e = launch_polar_keys(a, dtype, key_bits, s);
    if (e != hipSuccess) return e;
    switch (val_bits) {
      case 2: return values_mode<2>(a, dtype, val_mode, s);
      case 3: return values_mode<3>(a, dtype, val_mode, s);
      case 4: return values_mode<4>(a, dtype, val_mode, s);
    }
    return hipErrorInvalidValue;
  }
  if (key_mode == TQ_KEY_FP8) {
    if (key_bits != 8 || val_mode != TQ_VAL_UNIFORM) return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>((a.num_tokens * a.hkv + 3) / 4, 8192));
    const bool bf = dtype == TQ_BF16;
    switch (val_bits) {
      case 2: if (bf) hipLaunchKernelGGL((append_fp8_kernel<2, true>), grid, dim3(256), 0, s, a);
              else hipLaunchKernelGGL((append_fp8_kernel<2, false>), grid, dim3(256), 0, s, a); break;
      case 3: if (bf) hipLaunchKernelGGL((append_fp8_kernel<3, true>), grid, dim3(256), 0, s, a);
              else hipLaunchKernelGGL((append_fp8_kernel<3, false>), grid, dim3(256), 0, s, a); break;
      case 4: if (bf) hipLaunchKernelGGL((append_fp8_kernel<4, true>), grid, dim3(256), 0, s, a);
              else hipLaunchKernelGGL((append_fp8_kernel<4, false>), grid, dim3(256), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // bf16 inputs and uniform values: one launch for keys and values; the other
  // combinations take the per-vector kernels.
  if (dtype == TQ_BF16 && val_mode == TQ_VAL_UNIFORM && a.unit_grid_ok &&
      (a.num_tokens + 15) / 16 * a.hkv < ((int64_t)1 << 31)) {
    const bool qjl = key_mode == TQ_KEY_LLOYD_QJL;
    switch (key_bits) {
      case 2: return qjl ? page_vb<2, true>(a, val_bits, s) : page_vb<2, false>(a, val_bits, s);
      case 3: return qjl ? page_vb<3, true>(a, val_bits, s) : page_vb<3, false>(a, val_bits, s);
      case 4: return qjl ? page_vb<4, true>(a, val_bits, s) : page_vb<4, false>(a, val_bits, s);
    }
    return hipErrorInvalidValue;
  }
  hipError_t e;
  switch (key_bits) {
    case 8: e = keys_for_dtype<8, false>(a, dtype, s); break;   // 8-bit Lloyd-Max keys (no QJL)
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
