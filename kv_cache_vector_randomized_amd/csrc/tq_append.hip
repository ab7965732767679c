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

// ---------------------------------------------------------------------------
// Keys and values of whole pages, bf16 inputs (Lloyd-Max keys without QJL,
// uniform values).  One wave per group of 16 consecutive tokens of one KV head:
// when their slots are the 16 slots of one page in order (prefill), the wave
// assembles the page's fields in LDS and writes each with one contiguous
// 16-byte store per lane; otherwise every token goes to its own slot.
//
// Rotation on the matrix cores: with c = 16*ch + cl and k = 16*kh + kl, the
// Sylvester matrix factors as H[c][k] = H8[ch][kh] * H16[cl][kl].  The bf16 MFMA
// (16x16x16, fp32 sums) applies H16 to every 16-coordinate block of the 16
// tokens' sign-flipped rows (exact bf16 operands); H8 over the 8 blocks is then
// a 24-add butterfly in each lane, whose registers hold the 8 blocks of one
// column.  Lane (j, g) = (lane % 16, lane / 16) ends with coordinates 16*ch + j
// of tokens 4g..4g+3.
// ---------------------------------------------------------------------------
typedef short shortx4 __attribute__((ext_vector_type(4)));

// Sum or max of 4 values over the 16 lanes of each row (every lane gets it).
template <bool MAX>
__device__ __forceinline__ float row_reduce(float v) {
#define TQ_RSTEP(CTL)                                                                         \
  {                                                                                           \
    const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTL, 0xF, 0xF, false)); \
    v = MAX ? fmaxf(v, p) : v + p;                                                            \
  }
  TQ_RSTEP(0xB1) TQ_RSTEP(0x4E) TQ_RSTEP(0x141) TQ_RSTEP(0x140)
#undef TQ_RSTEP
  return v;
}
__device__ __forceinline__ float row_min(float v) {
  return -row_reduce<true>(-v);
}

// Codes of the 32 coordinates 32q..32q+31 (one byte each) packed LSB-first into
// B dwords (4*B bytes of the row).
template <int B>
__device__ __forceinline__ void pack32(const uint4 (&cb)[2], uint32_t (&w)[B]) {
  const uint32_t x[8] = {cb[0].x, cb[0].y, cb[0].z, cb[0].w, cb[1].x, cb[1].y, cb[1].z, cb[1].w};
  if constexpr (B == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t y0 = x[2 * i] | (x[2 * i] >> 4), y1 = x[2 * i + 1] | (x[2 * i + 1] >> 4);
      w[i] = __builtin_amdgcn_perm(y1, y0, 0x06040200u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t code = (x[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      const int bit = B * i, wi = bit >> 5, sh = bit & 31;
      w[wi] |= code << sh;
      if (sh + B > 32) w[wi + 1] |= code >> (32 - sh);
    }
  }
}

template <int KB, int VB>
__global__ __launch_bounds__(128) void append_page_kernel(AppendArgs a) {
  constexpr int KROW = 16 * KB;            // bytes of a packed key row
  constexpr int VROW = 16 * VB;            // bytes of a packed value row (= planes)
  // Wave 0 quantizes the 16 keys, wave 1 the 16 values of the group; each uses
  // only its own LDS, so the two never wait for each other.
  __shared__ QLut lut[kLutCells];
  __shared__ __align__(16) uint8_t kcode[16][kDim];       // key codes, one byte each [token][coord]
  __shared__ __align__(16) uint8_t vplane[64][16];        // value planes [plane][token]
  __shared__ float knorm_s[16], vmin_s[16], vsc_s[16];

  const int lane = threadIdx.x & 63;
  const bool keys = threadIdx.x < 64;
  const int j = lane & 15, g = lane >> 4;
  const int64_t grp = blockIdx.x;
  const int h = (int)(grp % a.hkv);
  const int64_t t0 = (grp / a.hkv) * 16;
  const int64_t tmax = a.num_tokens - 1;
  const uint16_t* kin = static_cast<const uint16_t*>(a.k);
  const uint16_t* vin = static_cast<const uint16_t*>(a.v);
  auto row_of = [&](int v) -> int64_t { return (min(t0 + v, tmax) * a.hkv + h) * kDim; };
  auto page_of = [&](int64_t s) -> uint8_t* { return a.cache + ((s >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes; };

  if (keys) {
    // inputs first, then the code grid, so the two latencies overlap
    uint2 ka[8];
    {
      const uint2* src = reinterpret_cast<const uint2*>(kin + row_of(j) + 4 * g);
#pragma unroll
      for (int kh = 0; kh < 8; ++kh) ka[kh] = src[4 * kh];
    }
    for (int i = lane; i < kLutCells; i += 64) lut[i] = a.c->klut[i];
    const int64_t tj = t0 + j;
    int64_t slot = tj <= tmax ? a.slots[tj] : -1;
    if (!(slot >= 0 && slot < a.num_blocks * kBlockTokensDev)) slot = -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- keys: signs, H16 on the matrix cores, H8 in registers
    shortx4 hb;                                  // B operand: H16[j][4g + e]
#pragma unroll
    for (int e = 0; e < 4; ++e) hb[e] = (__builtin_popcount(j & (4 * g + e)) & 1) ? (short)0xBF80 : (short)0x3F80;
    floatx4 z[8];
#pragma unroll
    for (int kh = 0; kh < 8; ++kh) {
      const int c0 = 16 * kh + 4 * g;            // first coordinate of this lane's 4 inputs
      const uint32_t sb = (a.sign_bits[c0 >> 5] >> (c0 & 31)) & 0xFu;
      uint2 x = ka[kh];
      x.x ^= ((sb & 1u) << 15) | ((sb & 2u) << 30);
      x.y ^= ((sb & 4u) << 13) | ((sb & 8u) << 28);
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      z[kh] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, x), hb, zero, 0, 0, 0);
    }
    // y[ch][r] = sum_kh H8[ch][kh] z[kh][r]: coordinate 16 ch + j of token 4g + r
#pragma unroll
    for (int len = 1; len < 8; len <<= 1)
#pragma unroll
      for (int i = 0; i < 8; i += 2 * len)
#pragma unroll
        for (int m = i; m < i + len; ++m) {
          const floatx4 p = z[m], q = z[m + len];
          z[m] = p + q;
          z[m + len] = p - q;
        }
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss[r] = fmaf(z[ch][r], z[ch][r], ss[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) ss[r] = row_reduce<false>(ss[r]);
    float cn2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // u = y / ||y||; a zero key gives u = 0, codes 2^(b-1) and norm 0
      const float inv = ss[r] > 0.f ? 1.f / sqrtf(ss[r]) : 0.f;
      float c2 = 0.f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        float c;
        const int code = lut_code(lut, z[ch][r] * inv, a.klut_scale, a.klut_bias, c);
        c2 = fmaf(c, c, c2);
        kcode[4 * g + r][16 * ch + j] = (uint8_t)code;
      }
      cn2[r] = c2;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cn2[r] = row_reduce<false>(cn2[r]);
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float n = sqrtf(ss[r]) * kInvSqrtDim;           // ||k|| (H/sqrt(d) is orthogonal)
        knorm_s[4 * g + r] = a.key_nc ? (n > 0.f ? n / sqrtf(cn2[r]) : 0.f) : n;
      }
    }


    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Key rows: lane l packs coordinates 32(l%4)..32(l%4)+31 of token l/4.
    const int kv = lane >> 2, kq = lane & 3;
    uint32_t kw[KB];
    {
      const uint4 cb[2] = {*reinterpret_cast<const uint4*>(&kcode[kv][32 * kq]),
                           *reinterpret_cast<const uint4*>(&kcode[kv][32 * kq + 16])};
      pack32<KB>(cb, kw);
    }
    const int64_t slot_kv = __builtin_amdgcn_ds_bpermute(kv << 2, (int)slot) |
                            ((int64_t)__builtin_amdgcn_ds_bpermute(kv << 2, (int)(slot >> 32)) << 32);
    if (slot_kv >= 0) {
      uint8_t* dst = page_of(slot_kv) + a.f.kcodes + (slot_kv & 15) * KROW + 4 * KB * kq;
      if constexpr (KB == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
      else if constexpr (KB == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(kw[0], kw[1]);
      else {
        uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
        d32[0] = kw[0]; d32[1] = kw[1]; d32[2] = kw[2];
      }
    }
    if (lane < 16 && slot >= 0) reinterpret_cast<float*>(page_of(slot) + a.f.knorm)[slot & 15] = knorm_s[lane];
  } else {
    uint4 va[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) va[p] = *reinterpret_cast<const uint4*>(vin + row_of(4 * p + g) + 8 * j);
    const int64_t tj = t0 + j;
    int64_t slot = tj <= tmax ? a.slots[tj] : -1;
    const bool ok = slot >= 0 && slot < a.num_blocks * kBlockTokensDev;
    if (!ok) slot = -1;
    const int64_t slot0 = __builtin_amdgcn_readfirstlane((int)slot) |
                          ((int64_t)__builtin_amdgcn_readfirstlane((int)(slot >> 32)) << 32);
    // the 16 tokens fill one page in order
    const bool whole = (__ballot(!(ok && slot == slot0 + j)) == 0ull) && slot0 >= 0 && (slot0 & 15) == 0;

    // ---- values: row g takes token 4p + g in pass p; lane j holds coordinates 8j..8j+7
    constexpr float levels = (float)((1 << VB) - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int v = 4 * p + g;
      const uint32_t wv[4] = {va[p].x, va[p].y, va[p].z, va[p].w};
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16lo(wv[i]);
        x[2 * i + 1] = bf16hi(wv[i]);
      }
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
      }
      mn = row_min(mn);
      mx = row_reduce<true>(mx);
      const float sc = (mx - mn) / levels;                  // correctly rounded division
      const float inv = sc > 0.f ? 1.f / sc : 0.f;
      // code = rint(fl32((x - mn) / sc)); the reciprocal product is within 2 ulp of the
      // correctly rounded quotient, so only values within 2^-18 of a rounding boundary
      // need the exact division
      float xq[8];
      uint32_t near = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xq[i] = (x[i] - mn) * inv;
        if (fabsf(xq[i] - floorf(xq[i]) - 0.5f) < 3.814697265625e-06f) near |= 1u << i;
      }
      if (near) {                                           // rare: exact quotients
#pragma unroll 1
        for (int i = 0; i < 8; ++i)
          if (near & (1u << i)) {
            float d = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) d = (m == i) ? x[m] - mn : d;
            const float qe = d / sc;
#pragma unroll
            for (int m = 0; m < 8; ++m) xq[m] = (m == i) ? qe : xq[m];
          }
      }
      uint32_t w = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= (uint32_t)fminf(rintf(xq[i]), levels) << (VB * i);   // half to even
      // bytes VB*j .. VB*j + VB - 1 of the row are planes VB*j + i
#pragma unroll
      for (int i = 0; i < VB; ++i) vplane[VB * j + i][v] = (uint8_t)(w >> (8 * i));
      if (j == 0) {
        vmin_s[v] = mn;
        vsc_s[v] = sc;
      }
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < 16 && slot >= 0) {
      uint8_t* pg = page_of(slot);
      reinterpret_cast<float*>(pg + a.f.vmin)[slot & 15] = vmin_s[lane];
      reinterpret_cast<float*>(pg + a.f.vscale)[slot & 15] = vsc_s[lane];
    }
    // Value planes: a whole page takes one 16-byte store per plane; otherwise
    // each token's byte of each plane goes to its own slot.
    if (whole) {
      if (lane < VROW)
        *reinterpret_cast<uint4*>(page_of(slot0) + a.f.vcodes + 16 * lane) =
            *reinterpret_cast<const uint4*>(&vplane[lane][0]);
    } else {
#pragma unroll 1
      for (int v = 0; v < 16; ++v) {
        const int64_t sv = __builtin_amdgcn_readlane((int)slot, v) |
                           ((int64_t)__builtin_amdgcn_readlane((int)(slot >> 32), v) << 32);
        if (sv >= 0 && lane < VROW) page_of(sv)[a.f.vcodes + 16 * lane + (sv & 15)] = vplane[lane][v];
      }
    }
  }
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

template <int KB>
hipError_t page_vb(const AppendArgs& a, int val_bits, hipStream_t s) {
  const dim3 grid((unsigned)((a.num_tokens + 15) / 16 * a.hkv));
  switch (val_bits) {
    case 2: hipLaunchKernelGGL((append_page_kernel<KB, 2>), grid, dim3(128), 0, s, a); break;
    case 3: hipLaunchKernelGGL((append_page_kernel<KB, 3>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((append_page_kernel<KB, 4>), grid, dim3(128), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dtype, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s) {
  // bf16 inputs, Lloyd-Max keys without QJL and uniform values: one launch for
  // both; the other combinations take the per-vector kernels.
  if (dtype == TQ_BF16 && key_mode != TQ_KEY_LLOYD_QJL && val_mode == TQ_VAL_UNIFORM) {
    switch (key_bits) {
      case 2: return page_vb<2>(a, val_bits, s);
      case 3: return page_vb<3>(a, val_bits, s);
      case 4: return page_vb<4>(a, val_bits, s);
    }
    return hipErrorInvalidValue;
  }
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
