// Generic path for gfx950: head_dim 64 or 256 and up to 16 query heads per KV
// head, the head sizes the tuned kernels (head_dim 128) do not take.  Same page
// format and the
// same results as the tuned path up to the decision band and the fp32 summation
// order; the aim is a plain structure, not speed:
//   * append and dequantize: one wave per (token, KV head) vector, lane l holding
//     coordinates l*M .. l*M + M - 1 (M = d / 64); the rotation is the in-register
//     butterfly over the low log2(M) bits and lane shuffles over the other six;
//   * decode: a work-group per (split, KV head, sequence), a token per lane for
//     the logits, a coordinate group per lane for the value sums, and a second
//     launch that merges the splits by log-sum-exp.
// The method: issoh.co.jp "TurboQuantとは？…", 第1段 (random rotation, Lloyd-Max
// codes of the unit vector, norm kept apart) and 第2段 (uniform values with a
// per-vector min and scale); lilting.ch TurboQuant article, QJL section (signs of
// S r of the residual, the corrected score); turboquant-vllm write-up, "Bugs
// Nobody Else Has Found" (fp32 norms, attention over the compressed cache).
#include <algorithm>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kGenWaves = 4;   // waves per work-group
constexpr float kGenLog2e = 1.4426950408889634f;
constexpr float kGenLn2 = 0.6931471805599453f;

// Lane l's copy of the value of lane l ^ m.  m = 1 and 2 are quad permutations,
// m = 4 the half-row mirror (l ^ 7) followed by the quad reversal (^ 3), m = 8
// the row mirror (l ^ 15) followed by the half-row mirror (^ 7): DPP moves within
// a row of 16 lanes.  m = 16 and 32 go through the LDS crossbar.  (m is a constant
// once the callers' loops are unrolled, and the other branches fold away.)
template <int CTRL>
__device__ __forceinline__ uint32_t gdpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t gxor(uint32_t v, int m) {
  if (m == 1) return gdpp<0xB1>(v);                    // quad_perm [1,0,3,2]
  if (m == 2) return gdpp<0x4E>(v);                    // quad_perm [2,3,0,1]
  if (m == 4) return gdpp<0x1B>(gdpp<0x141>(v));       // row_half_mirror, quad_perm [3,2,1,0]
  if (m == 8) return gdpp<0x141>(gdpp<0x140>(v));      // row_mirror, row_half_mirror
  return (uint32_t)__shfl_xor((int)v, m);
}
__device__ __forceinline__ float gxor(float v, int m) { return __uint_as_float(gxor(__float_as_uint(v), m)); }
__device__ __forceinline__ double gxor(double v, int m) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = gxor((uint32_t)b, m), hi = gxor((uint32_t)(b >> 32), m);
  return __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ __forceinline__ float gw_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += gxor(v, m);
  return v;
}
__device__ __forceinline__ double gw_sum64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += gxor(v, m);
  return v;
}
__device__ __forceinline__ float gw_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, gxor(v, m));
  return v;
}
__device__ __forceinline__ float gw_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, gxor(v, m));
  return v;
}

// 1 / sqrt(d) of the normalized transform
template <int D>
__host__ __device__ constexpr double inv_sqrt_dim() {
  return D == 64 ? 0.125 : D == 256 ? 0.0625 : 0.08838834764831844;
}

// Unnormalized Sylvester (natural order) Walsh-Hadamard transform of a vector whose
// coordinate l*M + i sits in x[i] of lane l: coordinate bits below log2(M) pair
// within a lane, the six above pair lane l with lane l ^ m.  The element whose bit
// is set takes (other - own), the other one (own + other).
template <int M, typename T>
__device__ __forceinline__ void gen_fwht(T (&x)[M], int lane) {
#pragma unroll
  for (int len = 1; len < M; len <<= 1)
#pragma unroll
    for (int i = 0; i < M; i += 2 * len)
#pragma unroll
      for (int j = i; j < i + len; ++j) {
        const T u = x[j], w = x[j + len];
        x[j] = u + w;
        x[j + len] = u - w;
      }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const T p = gxor(x[i], m);
      x[i] = upper ? p - x[i] : x[i] + p;
    }
  }
}

// This lane's coordinates of row `row` of a [rows][d] activation array (bf16 or fp32).
// (one vector load per lane when the array is 16-byte aligned -- M bf16 values
// are 2, 4 or 8 bytes, M fp32 values 4, 8 or 16 and rows are whole multiples of
// 16 bytes -- else one load per value)
template <int M>
__device__ __forceinline__ void gen_load(const void* base, int64_t row, bool bf16, int lane, float (&x)[M]) {
  constexpr int D = 64 * M;
  const bool vec = ((uintptr_t)base & 15u) == 0;
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row * D + lane * M;
    if (vec && M > 1) {
      uint32_t w[(M + 1) / 2];
      if constexpr (M == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
      } else if constexpr (M == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        w[0] = u.x;
        w[1] = u.y;
      }
#pragma unroll
      for (int i = 0; i < M; ++i) x[i] = __uint_as_float(i & 1 ? w[i / 2] & 0xffff0000u : w[i / 2] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < M; ++i) x[i] = __uint_as_float((uint32_t)p[i] << 16);
    }
  } else {
    const float* p = static_cast<const float*>(base) + row * D + lane * M;
    if (vec && M == 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      x[0] = u.x;
      x[1] = u.y;
      x[2] = u.z;
      x[3] = u.w;
    } else if (vec && M == 2) {
      const float2 u = *reinterpret_cast<const float2*>(p);
      x[0] = u.x;
      x[1] = u.y;
    } else {
#pragma unroll
      for (int i = 0; i < M; ++i) x[i] = p[i];
    }
  }
}

// The raw words of lane's M coordinates of a row (bf16 bits or fp32 bits), loads
// only, so that several rows can be requested before any of them is waited for.
template <int M>
__device__ __forceinline__ void gen_fetch(const void* base, int64_t row, bool bf16, int lane, uint32_t (&w)[M]) {
  constexpr int D = 64 * M;
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row * D + lane * M;
#pragma unroll
    for (int i = 0; i < M; ++i) w[i] = p[i];
  } else {
    const uint32_t* p = static_cast<const uint32_t*>(base) + row * D + lane * M;
#pragma unroll
    for (int i = 0; i < M; ++i) w[i] = p[i];
  }
}
template <int M>
__device__ __forceinline__ void gen_cvt(const uint32_t (&w)[M], bool bf16, float (&x)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) x[i] = __uint_as_float(bf16 ? w[i] << 16 : w[i]);
}

// code = #{j : t_j <= y} over the 2^bits - 1 ascending thresholds t (binary search:
// each step keeps the count of thresholds known to be <= y).
__device__ __forceinline__ int gen_code(const float* t, int bits, double y) {
  int n = 0;
  for (int step = 1 << (bits - 1); step >= 1; step >>= 1)
    if ((double)t[n + step - 1] <= y) n += step;
  return n;
}

// Byte p of the LSB-first bit stream of n codes of `bits` bits held one per byte.
__device__ __forceinline__ uint32_t gen_stream_byte(const uint8_t* codes, int n, int bits, int p) {
  uint32_t v = 0u;
  for (int i = (8 * p) / bits; i < n && bits * i < 8 * p + 8; ++i) {
    const int sh = bits * i - 8 * p;
    const uint32_t c = codes[i];
    v |= sh >= 0 ? (c << sh) : (c >> -sh);
  }
  return v & 0xFFu;
}

// Code i of an LSB-first packed row whose byte p sits at row[stride * p]
// (stride 1: slot-major key rows; 16: plane-major value rows).
__device__ __forceinline__ uint32_t gen_read_code(const uint8_t* row, int stride, int bits, int i) {
  const int bit = bits * i, byte = bit >> 3, sh = bit & 7;
  uint32_t v = row[stride * byte];
  if (sh + bits > 8) v |= (uint32_t)row[stride * (byte + 1)] << 8;
  return (v >> sh) & ((1u << bits) - 1u);
}

// Make a wave's LDS writes visible to its later LDS reads.
__device__ __forceinline__ void gen_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Quantize-append: one wave per (token, KV head).  FP8 keys: the E4M3 byte of each
// coordinate.  Lloyd-Max keys: ||k|| and the rotation in
// fp64 (the squares of fp32 or bf16 values are exact there), codes of the unit
// coordinate, the stored norm (plain or corrected) rounded once to fp32, and for
// QJL keys the residual r = y - norm * C[code] in the rotated frame, its norm and
// the signs of S r (fp64 sums of fp32 S).  Values: uniform (min, scale =
// fl32((max - min) / (2^b - 1)), code = rint((v - min) / scale) with the quotient
// in fp64) or Lloyd-Max as the keys with a plain norm.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kGenWaves) void gen_append_kernel(GenAppendArgs a) {
  constexpr int M = D / 64;
  constexpr double isd = inv_sqrt_dim<D>();
  __shared__ float s_kt[256], s_kc[256], s_vt[16];
  __shared__ uint8_t s_codes[kGenWaves][D];
  __shared__ double s_r[kGenWaves][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 256; i += 64 * kGenWaves) {
    s_kt[i] = a.c->kt[i];
    s_kc[i] = a.c->kc[i];
  }
  if (tid < 16) s_vt[tid] = a.c->vt[tid];
  __syncthreads();
  float sg[M];
#pragma unroll
  for (int i = 0; i < M; ++i) sg[i] = a.c->signs[lane * M + i];

  const int64_t nvec = a.num_tokens * a.hkv;
  for (int64_t vi = (int64_t)blockIdx.x * kGenWaves + wave; vi < nvec; vi += (int64_t)gridDim.x * kGenWaves) {
    const int64_t t = vi / a.hkv;
    const int h = (int)(vi - t * a.hkv);
    // the vector's key and value rows are requested with its slot, before any of
    // them is used: one round trip per vector instead of three
    uint32_t kw[M], vw[M];
    gen_fetch<M>(a.k, vi, BF16, lane, kw);
    gen_fetch<M>(a.v, vi, BF16, lane, vw);
    int64_t slot = -1;
    if (a.slots) {
      slot = a.slots[t];
    } else {
      // one-launch step: the new token of sequence t is position seq_lens[t] - 1
      int sl = a.seq_lens[t];
      sl = max(0, min(sl, min(a.max_seq, 16 * a.max_blocks)));
      if (sl > 0 && a.num_blocks > 0) {
        const int blk = a.block_tables[t * a.max_blocks + (sl - 1) / 16];
        if (blk >= 0 && blk < a.num_blocks) slot = (int64_t)blk * 16 + (sl - 1) % 16;
      }
    }
    if (slot < 0 || slot >= a.num_blocks * 16) continue;   // uniform over the wave
    uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
    const int so = (int)(slot & 15);

    float kf[M], vf[M];
    gen_cvt<M>(kw, BF16, kf);
    gen_cvt<M>(vw, BF16, vf);

    // ---- keys
    if (a.key_mode == 3) {
      // FP8 keys: the E4M3 byte of every coordinate, coordinate i at byte i; no norm
      uint8_t* krow = page + a.f.kcodes + so * a.rows.kcodes + lane * M;
#pragma unroll
      for (int i = 0; i < M; ++i) krow[i] = (uint8_t)fp8_e4m3(kf[i]);
    } else {
    double z[M], ss = 0.0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      ss = fma((double)kf[i], (double)kf[i], ss);
      z[i] = (double)kf[i] * (double)sg[i];
    }
    const double n = sqrt(gw_sum64(ss));
    gen_fwht<M, double>(z, lane);                  // z = H(s * k); y = z / sqrt(d)
    const double iu = n > 0.0 ? isd / n : 0.0;    // u = y / ||k|| (0 for a zero key)
    float cv[M];
    double cn2 = 0.0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int code = gen_code(s_kt, a.key_bits, z[i] * iu);
      s_codes[wave][lane * M + i] = (uint8_t)code;
      cv[i] = s_kc[code];
      cn2 = fma((double)cv[i], (double)cv[i], cn2);
    }
    cn2 = gw_sum64(cn2);
    const float norm = stored_norm(n, cn2, a.key_mode == 1);
    gen_wave_sync();
    for (int p = lane; p < (int)a.rows.kcodes; p += 64)
      page[a.f.kcodes + so * a.rows.kcodes + p] = (uint8_t)gen_stream_byte(s_codes[wave], D, a.key_bits, p);
    if (lane == 0) reinterpret_cast<float*>(page + a.f.knorm)[so] = norm;
    if (a.key_mode == 2) {
      double rr = 0.0;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const double r = z[i] * isd - (double)norm * (double)cv[i];
        s_r[wave][lane * M + i] = r;
        rr = fma(r, r, rr);
      }
      rr = gw_sum64(rr);
      gen_wave_sync();   // the residual is in LDS, the key bytes are read
      // rows lane*M + i of S r
      double pr[M];
#pragma unroll
      for (int i = 0; i < M; ++i) pr[i] = 0.0;
#pragma unroll 1
      for (int k0 = 0; k0 < D; k0 += 32 / M) {
        constexpr int SR = 32 / M;   // rows of S^T per batch, requested before they are used
        float sv[SR][M];
#pragma unroll
        for (int u = 0; u < SR; ++u)
#pragma unroll
          for (int i = 0; i < M; ++i) sv[u][i] = a.St[(k0 + u) * D + lane * M + i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SR; ++u) {
          const double rk = s_r[wave][k0 + u];
#pragma unroll
          for (int i = 0; i < M; ++i) pr[i] = fma((double)sv[u][i], rk, pr[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < M; ++i) s_codes[wave][lane * M + i] = pr[i] >= 0.0 ? 1 : 0;
      gen_wave_sync();
      for (int p = lane; p < (int)a.rows.ksigns; p += 64)
        page[a.f.ksigns + so * a.rows.ksigns + p] = (uint8_t)gen_stream_byte(s_codes[wave], D, 1, p);
      if (lane == 0) reinterpret_cast<float*>(page + a.f.kres)[so] = (float)sqrt(rr);
    }
    }
    gen_wave_sync();   // every read of s_codes is done before the values overwrite it

    // ---- values
    if (a.val_mode == 0) {
      float mn = vf[0], mx = vf[0];
#pragma unroll
      for (int i = 1; i < M; ++i) {
        mn = fminf(mn, vf[i]);
        mx = fmaxf(mx, vf[i]);
      }
      mn = gw_min(mn);
      mx = gw_max(mx);
      const int levels = (1 << a.val_bits) - 1;
      const float sc = (float)(((double)mx - (double)mn) / (double)levels);
#pragma unroll
      for (int i = 0; i < M; ++i) {
        double code = 0.0;
        if (sc > 0.f) code = fmin(fmax(rint(((double)vf[i] - (double)mn) / (double)sc), 0.0), (double)levels);
        s_codes[wave][lane * M + i] = (uint8_t)code;
      }
      if (lane == 0) {
        reinterpret_cast<float*>(page + a.f.vmin)[so] = mn;
        reinterpret_cast<float*>(page + a.f.vscale)[so] = sc;
      }
    } else {
      double zv[M], vs = 0.0;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        vs = fma((double)vf[i], (double)vf[i], vs);
        zv[i] = (double)vf[i] * (double)sg[i];
      }
      const double vnorm = sqrt(gw_sum64(vs));
      gen_fwht<M, double>(zv, lane);
      const double ivu = vnorm > 0.0 ? isd / vnorm : 0.0;
#pragma unroll
      for (int i = 0; i < M; ++i) s_codes[wave][lane * M + i] = (uint8_t)gen_code(s_vt, a.val_bits, zv[i] * ivu);
      if (lane == 0) reinterpret_cast<float*>(page + a.f.vmin)[so] = (float)vnorm;
    }
    gen_wave_sync();
    for (int p = lane; p < (int)a.rows.vcodes; p += 64)
      page[a.f.vcodes + 16 * p + so] = (uint8_t)gen_stream_byte(s_codes[wave], D, a.val_bits, p);
    gen_wave_sync();   // the next vector's codes overwrite s_codes
  }
}

// ---------------------------------------------------------------------------
// Decode attention, split part: work-group (split, KV head, sequence) takes tokens
// [split * chunk, (split + 1) * chunk) of the sequence, wave w the 64-token blocks
// w, w + 4, ...  Logits are base 2: the query rows are rotated and scaled by
// softmax_scale * log2(e) / sqrt(d), so logit_2 = norm * <q'', C[code]> (+ rho *
// <coef S q'', 2 sigma - 1> for QJL keys).  A lane takes one token of the block:
// its code row (KB bits per code, whole words) in registers, 32 centroids at a
// time, every head's dot product against the query rows in LDS.  Each lane reads
// the two value planes of each of the block's 4 pages that hold its M coordinates'
// codes, the value scalars go through LDS, and every lane adds the 64 weighted
// value rows for its M coordinates.  Each wave keeps a running max, sum
// and weighted value sum per head; the work-group's four are merged through LDS
// and stored as the split's partial (max, sum, d sums) per head.
// Dynamic LDS of the decode work-group, sized for the group and value width at
// launch: the query rows, their QJL projections, the softmax weights of each
// wave's block, the wave partials and the value scalars.
// With the logits on the matrix cores (`mf`), also the A operands of every K step
// and the centroid-term table of every code byte.
struct GenDecodeLds {
  int q, p, w, part, v, vs, qa, kt2, bytes;
};
typedef _Float16 genhalf8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 gen_mfma_f16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(genhalf8, a), __builtin_bit_cast(genhalf8, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ uint32_t gen_pack_f16(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
__host__ __device__ inline GenDecodeLds gen_decode_lds(int d, int group, bool qjl, int vrow, bool mf) {
  GenDecodeLds L;
  L.q = 0;
  L.p = L.q + 4 * group * d;
  L.w = L.p + (qjl ? 4 * group * d : 0);
  L.part = L.w + 4 * kGenWaves * group * 64;
  L.v = L.part + 4 * kGenWaves * (2 + d);
  L.v = (L.v + 15) & ~15;
  L.vs = L.v;   // (value planes are read straight into registers)
  L.qa = L.vs + 4 * kGenWaves * 2 * 64;
  L.kt2 = L.qa + (mf ? ((group + 3) / 4) * (d / 16) * 64 * 16 : 0);
  L.bytes = L.kt2 + (mf ? 256 * 16 : 0);
  return L;
}

template <int D, int KB, int GM>
__global__ __launch_bounds__(64 * kGenWaves) __attribute__((amdgpu_waves_per_eu(GM <= 4 ? 3 : 2)))
void gen_decode_kernel(GenDecodeArgs a) {
  constexpr int M = D / 64;
  constexpr int NW = KB * D / 32;        // words of a key code row
  constexpr int NS = D / 32;             // words of a sign row
  constexpr float isd = (float)inv_sqrt_dim<D>();
  extern __shared__ __align__(16) unsigned char gsm[];
  __shared__ float s_kc[256], s_vc[16];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int hq = a.hkv * G;
  const int vrow = (int)a.rows.vcodes;
  constexpr bool MF = KB == 4 || KB == 2;   // 4- and 2-bit codes: logits on the f16 matrix cores
  constexpr int NRB = GM / 4;          // row blocks of 4 heads in the register arrays
  const int nrb = (G + 3) / 4;         // row blocks in use
  const GenDecodeLds L = gen_decode_lds(D, G, a.key_mode == 2, vrow, MF);
  float* s_q = reinterpret_cast<float*>(gsm + L.q);                      // [G][D]
  float* s_p = reinterpret_cast<float*>(gsm + L.p);                      // [G][D] (QJL)
  float* s_w = reinterpret_cast<float*>(gsm + L.w) + wave * G * 64;      // this wave's [G][64]
  float* s_part = reinterpret_cast<float*>(gsm + L.part);                // [waves][2 + D]
  float* s_vs = reinterpret_cast<float*>(gsm + L.vs) + wave * 2 * 64;    // this wave's [2][64]
  for (int i = tid; i < 256; i += 64 * kGenWaves) s_kc[i] = a.c->kc[i];
  if (tid < 16) s_vc[tid] = a.c->vc[tid];
  for (int h = wave; h < G; h += kGenWaves) {
    float x[M];
    gen_load<M>(a.q, (int64_t)b * hq + (int64_t)kvh * G + h, a.q_bf16 != 0, lane, x);
    // FP8 keys are stored unrotated: their query rows are only scaled
    const bool rot = a.key_mode != 3;
    if (rot) {
#pragma unroll
      for (int i = 0; i < M; ++i) x[i] *= a.c->signs[lane * M + i];
      gen_fwht<M, float>(x, lane);
    }
    const float f = a.scale * (rot ? isd : 1.f) * kGenLog2e;
#pragma unroll
    for (int i = 0; i < M; ++i) s_q[h * D + lane * M + i] = x[i] * f;
  }
  __syncthreads();
  const bool qjl = a.key_mode == 2;
  if (qjl) {
    for (int h = wave; h < G; h += kGenWaves) {
      float acc[M];
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = 0.f;
#pragma unroll 1
      for (int k0 = 0; k0 < D; k0 += 32 / M) {
        constexpr int SR = 32 / M;   // rows of S^T per batch, requested before they are used
        float sv[SR][M];
#pragma unroll
        for (int u = 0; u < SR; ++u)
#pragma unroll
          for (int i = 0; i < M; ++i) sv[u][i] = a.St[(k0 + u) * D + lane * M + i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SR; ++u) {
          const float qk = s_q[h * D + k0 + u];
#pragma unroll
          for (int i = 0; i < M; ++i) acc[i] = fmaf(sv[u][i], qk, acc[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < M; ++i) s_p[h * D + lane * M + i] = acc[i] * a.qjl_coef;
    }
    __syncthreads();
  }

  // Logits on the f16 matrix cores (4- and 2-bit codes).  Rows of the A operand of row
  // block rb are (head 4rb + h, term t) = 4h + t: the head's rotated query row
  // times 2^s1 split into three f16 terms (row 4h + 3 is zero).  In K step ks the K slots
  // 2i and 2i + 1 of lane (m, kg) (m = lane % 16, kg = lane / 16) hold coordinate
  // kg*D/4 + 4ks + i, against the two f16 terms (hi, lo) of that coordinate's
  // centroid times 2^s2 in the B operand, so a lane's four codes of a K step are
  // two consecutive bytes (4-bit codes) or one byte (2-bit codes) of its token's
  // code row, turned into B through a table of the centroid terms of each code
  // byte.  Products carry about 22 significant
  // bits; the A operands of every K step are built once per work-group in LDS.
  __shared__ int s_s1[MF ? kGenMaxGroup : 1];   // 2^s1[h]: head h's query scale
  int s2 = 0;
  if constexpr (MF) {
    uint4* s_qa = reinterpret_cast<uint4*>(gsm + L.qa);
    float cm = 0.f;
#pragma unroll
    for (int c = 0; c < (1 << KB); ++c) cm = fmaxf(cm, fabsf(s_kc[c]));
    s2 = cm > 0.f ? 14 - __builtin_amdgcn_frexp_expf(cm) : 0;
    // per code byte, the (hi, lo) f16 terms of its codes' centroids in stream order:
    // two codes (8 bytes) for 4-bit codes, four (16 bytes) for 2-bit codes
    constexpr int PER = 8 / KB;
    for (int i = tid; i < 256; i += 64 * kGenWaves) {
      uint32_t e[4];
#pragma unroll
      for (int hh = 0; hh < PER; ++hh) {
        const float y = ldexpf(s_kc[(i >> (KB * hh)) & ((1 << KB) - 1)], s2);
        const _Float16 hi = (_Float16)y;
        e[hh] = gen_pack_f16(hi, (_Float16)(y - (float)hi));
      }
      if constexpr (KB == 4) reinterpret_cast<uint2*>(gsm + L.kt2)[i] = make_uint2(e[0], e[1]);
      else reinterpret_cast<uint4*>(gsm + L.kt2)[i] = make_uint4(e[0], e[1], e[2], e[3]);
    }
    for (int h = wave; h < G; h += kGenWaves) {
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < M; ++i) mx = fmaxf(mx, fabsf(s_q[h * D + lane * M + i]));
      mx = gw_max(mx);
      if (lane == 0) s_s1[h] = mx > 0.f ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
    }
    __syncthreads();
    const int m = lane & 15, kg = lane >> 4, tA = m & 3;
    for (int idx = wave; idx < nrb * (D / 16); idx += kGenWaves) {
      const int rb = idx / (D / 16), ks = idx - rb * (D / 16);
      const int hA = 4 * rb + (m >> 2);
      const int s1a = hA < G ? s_s1[hA] : 0;
      uint32_t dw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dw[i] = 0u;
        if (hA < G && tA < 3) {
          const float x = ldexpf(s_q[hA * D + kg * (D / 4) + 4 * ks + i], s1a);
          const _Float16 q0 = (_Float16)x;
          const float r1 = x - (float)q0;
          const _Float16 q1 = (_Float16)r1;
          const _Float16 q2 = (_Float16)(r1 - (float)q1);
          const _Float16 qt = tA == 0 ? q0 : tA == 1 ? q1 : q2;
          dw[i] = gen_pack_f16(qt, qt);
        }
      }
      s_qa[idx * 64 + lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    }
    __syncthreads();
  }

  int seq_len = a.seq_lens[b];
  seq_len = max(0, min(seq_len, min(a.max_seq, 16 * a.max_blocks)));
  if (a.num_blocks <= 0) seq_len = 0;
  const int t0 = split * a.chunk;
  const int t1 = min(t0 + a.chunk, seq_len);
  const int64_t pstride = a.f.page_bytes;

  float m_run[GM], l_run[GM], o[GM][M];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) o[h][i] = 0.f;
  }
  for (int tb = t0 + 64 * wave; tb < t1; tb += 64 * kGenWaves) {
    const int t = tb + lane;
    int blk = -1;
    if (t < t1) blk = a.block_tables[(int64_t)b * a.max_blocks + t / 16];
    const bool valid = t < t1 && blk >= 0 && blk < a.num_blocks;
    const int so = t & 15;
    const uint8_t* page = a.cache + ((int64_t)(valid ? blk : 0) * a.hkv + kvh) * pstride;
    float lg[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) lg[h] = -INFINITY;
    float dm[GM];    // matrix-core dot products of this lane's token, per head
    if constexpr (MF) {
      // tile ct = page ct of the block (tokens tb + 16ct .. + 15): lane (n, kg) reads
      // bytes kg*D/8 .. (kg+1)*D/8 - 1 of token 16ct + n's code row (a page with no
      // valid token reads block 0's: in range, and its dot products are not used)
      const uint64_t vm = __ballot(valid);
      const uint2* s_kt2 = reinterpret_cast<const uint2*>(gsm + L.kt2);   // 4-bit codes
      const uint4* s_kt4 = reinterpret_cast<const uint4*>(gsm + L.kt2);   // 2-bit codes
      const uint4* s_qa = reinterpret_cast<const uint4*>(gsm + L.qa);
      const int n = lane & 15, kg = lane >> 4;
      constexpr int QW = D * KB / 128;   // dwords of a quarter row
      uint32_t qr[4][QW];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int bc = __builtin_amdgcn_readlane(blk, 16 * ct);
        const bool tv = ((vm >> (16 * ct)) & 0xFFFFull) != 0;
        const uint8_t* rp = a.cache + ((int64_t)(tv ? bc : 0) * a.hkv + kvh) * pstride + a.f.kcodes +
                            n * (D * KB / 8) + kg * (4 * QW);
        if constexpr (QW >= 4) {
#pragma unroll
          for (int j = 0; j < QW / 4; ++j) {
            const uint4 u = reinterpret_cast<const uint4*>(rp)[j];
            qr[ct][4 * j] = u.x; qr[ct][4 * j + 1] = u.y; qr[ct][4 * j + 2] = u.z; qr[ct][4 * j + 3] = u.w;
          }
        } else if constexpr (QW == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(rp);
          qr[ct][0] = u.x; qr[ct][1] = u.y;
        } else {
          qr[ct][0] = *reinterpret_cast<const uint32_t*>(rp);
        }
      }
      floatx4 acc[NRB][4];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rb][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        uint4 A[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          if (NRB == 1 || rb < nrb) A[rb] = s_qa[(rb * (D / 16) + ks) * 64 + lane];   // uniform
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          uint4 B;
          if constexpr (KB == 4) {   // the K step's four codes: two bytes
            const uint32_t two = (qr[ct][ks >> 1] >> (16 * (ks & 1))) & 0xFFFFu;
            const uint2 e0 = s_kt2[two & 0xFFu], e1 = s_kt2[two >> 8];
            B = make_uint4(e0.x, e0.y, e1.x, e1.y);
          } else {                   // one byte
            B = s_kt4[(qr[ct][ks >> 2] >> (8 * (ks & 3))) & 0xFFu];
          }
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            if (NRB == 1 || rb < nrb) acc[rb][ct] = gen_mfma_f16(A[rb], B, acc[rb][ct]);   // uniform
        }
      }
      // lane (n, h) of row block rb holds head 4rb + h's dot product for token
      // 16ct + n: through s_w to the token's lane (the previous block's weights in
      // s_w are no longer read)
      const float sc2 = ldexpf(1.f, -s2);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int hO = 4 * rb + (lane >> 4);
        if ((NRB == 1 || rb < nrb) && hO < G) {
          const float sc1 = ldexpf(1.f, -s_s1[hO]);   // two steps: neither underflows alone
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            s_w[hO * 64 + 16 * ct + n] = ((acc[rb][ct][0] + acc[rb][ct][1] + acc[rb][ct][2]) * sc2) * sc1;
        }
      }
      gen_wave_sync();
#pragma unroll
      for (int h = 0; h < GM; ++h) dm[h] = h < G ? s_w[h * 64 + lane] : 0.f;
    }
    float vs0 = 0.f, vs1 = 0.f;
    if (valid) {
      const float norm = a.key_mode == 3 ? 1.f : reinterpret_cast<const float*>(page + a.f.knorm)[so];   // FP8: no norm
      float dot[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) dot[h] = MF ? dm[h] : 0.f;
      if constexpr (!MF) {
      uint32_t w[NW];
      const uint2* kr = reinterpret_cast<const uint2*>(page + a.f.kcodes + so * (4 * NW));
#pragma unroll
      for (int j = 0; j < NW / 2; ++j) {
        const uint2 u2 = kr[j];
        w[2 * j] = u2.x;
        w[2 * j + 1] = u2.y;
      }
#pragma unroll
      for (int c0 = 0; c0 < D; c0 += 32) {
        float cv[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) cv[j] = s_kc[get_code<KB>(w, c0 + j)];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h < G) {
            float acc = dot[h];
#pragma unroll
            for (int j = 0; j < 32; j += 4) {
              const float4 qv = *reinterpret_cast<const float4*>(&s_q[h * D + c0 + j]);
              acc = fmaf(qv.x, cv[j], acc);
              acc = fmaf(qv.y, cv[j + 1], acc);
              acc = fmaf(qv.z, cv[j + 2], acc);
              acc = fmaf(qv.w, cv[j + 3], acc);
            }
            dot[h] = acc;
          }
        }
      }
      }   // !MF
#pragma unroll
      for (int h = 0; h < GM; ++h) lg[h] = norm * dot[h];
      if (qjl) {
        const float rho = reinterpret_cast<const float*>(page + a.f.kres)[so];
        uint32_t sw[NS];
        const uint2* sr = reinterpret_cast<const uint2*>(page + a.f.ksigns + so * (4 * NS));
#pragma unroll
        for (int j = 0; j < NS / 2; ++j) {
          const uint2 u2 = sr[j];
          sw[2 * j] = u2.x;
          sw[2 * j + 1] = u2.y;
        }
        float cs[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) cs[h] = 0.f;
#pragma unroll
        for (int c0 = 0; c0 < D; c0 += 32) {
          const uint32_t bits = sw[c0 / 32];
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            if (h < G) {
              float acc = cs[h];
#pragma unroll
              for (int j = 0; j < 32; j += 4) {
                const float4 pv = *reinterpret_cast<const float4*>(&s_p[h * D + c0 + j]);
                acc += ((bits >> j) & 1u) ? pv.x : -pv.x;
                acc += ((bits >> (j + 1)) & 1u) ? pv.y : -pv.y;
                acc += ((bits >> (j + 2)) & 1u) ? pv.z : -pv.z;
                acc += ((bits >> (j + 3)) & 1u) ? pv.w : -pv.w;
              }
              cs[h] = acc;
            }
          }
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) lg[h] = fmaf(rho, cs[h], lg[h]);
      }
      if (a.logits != nullptr) {
#pragma unroll
        for (int h = 0; h < GM; ++h)
          if (h < G) a.logits[((int64_t)b * hq + (int64_t)kvh * G + h) * a.max_seq + t] = lg[h] * kGenLn2;
      }
      vs0 = reinterpret_cast<const float*>(page + a.f.vmin)[so];
      if (a.val_mode == 0) vs1 = reinterpret_cast<const float*>(page + a.f.vscale)[so];
    }
    s_vs[lane] = vs0;
    s_vs[64 + lane] = vs1;
    // the value planes of the block's four pages (page pg holds tokens tb + 16 pg ..
    // tb + 16 pg + 15, one block id; a page with no valid token is not read)
    const uint64_t vmask = __ballot(valid);
    int bpg[4];
    bool pvld[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      bpg[pg] = __shfl(blk, 16 * pg);
      pvld[pg] = ((vmask >> (16 * pg)) & 0xFFFFull) != 0;
    }
    // Lane l's value codes (coordinates l*M .. l*M + M - 1) are bits [l*M*b,
    // (l+1)*M*b) of a value row, which lie in two planes at most (M*b <= 16, whole
    // bytes when b = 4): each page's two planes hold them for its 16 tokens, read
    // from the cache here (16 bytes each), before the softmax needs the wave.
    const int vb = a.val_bits;
    const int vbit0 = lane * M * vb;
    const int q0 = vbit0 >> 3, vsh = vbit0 & 7;
    const int q1 = min(q0 + 1, vrow - 1);
    uint4 P0[4], P1[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      P0[pg] = P1[pg] = make_uint4(0u, 0u, 0u, 0u);
      if (pvld[pg]) {   // uniform
        const uint4* vp = reinterpret_cast<const uint4*>(a.cache + ((int64_t)bpg[pg] * a.hkv + kvh) * pstride +
                                                         a.f.vcodes);
        P0[pg] = vp[q0];
        P1[pg] = vp[q1];
      }
    }
    // online softmax of each head over the block's 64 tokens
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float mnew = fmaxf(m_run[h], gw_max(lg[h]));
        float p = 0.f;
        if (mnew != -INFINITY) {
          const float al = m_run[h] == -INFINITY ? 0.f : exp2f(m_run[h] - mnew);
          p = lg[h] == -INFINITY ? 0.f : exp2f(lg[h] - mnew);
          l_run[h] = fmaf(l_run[h], al, gw_sum(p));
#pragma unroll
          for (int i = 0; i < M; ++i) o[h][i] *= al;
          m_run[h] = mnew;
        }
        s_w[h * 64 + lane] = p;
      }
    }
    gen_wave_sync();
    // Values of the block's tokens: lane l adds coordinates l*M .. l*M + M - 1 from
    // the planes read above; the weights and value scalars are read four tokens at
    // a time.  Tokens that are not valid have weight 0 and scalars 0.
    {
      const int sh = vsh;
      const uint32_t cmask = (1u << vb) - 1u;
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
        if (!pvld[pg]) continue;   // uniform: no valid token in this page
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const int u0 = pg * 16 + 4 * t4;
          const float4 v0q = *reinterpret_cast<const float4*>(&s_vs[u0]);
          const float4 v1q = *reinterpret_cast<const float4*>(&s_vs[64 + u0]);
          const uint32_t w0 = t4 == 0 ? P0[pg].x : t4 == 1 ? P0[pg].y : t4 == 2 ? P0[pg].z : P0[pg].w;
          const uint32_t w1 = t4 == 0 ? P1[pg].x : t4 == 1 ? P1[pg].y : t4 == 2 ? P1[pg].z : P1[pg].w;
          float vh[4][M];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t word = ((w0 >> (8 * e)) & 0xFFu) | (((w1 >> (8 * e)) & 0xFFu) << 8);
            const float v0 = e == 0 ? v0q.x : e == 1 ? v0q.y : e == 2 ? v0q.z : v0q.w;
            const float v1 = e == 0 ? v1q.x : e == 1 ? v1q.y : e == 2 ? v1q.z : v1q.w;
#pragma unroll
            for (int i = 0; i < M; ++i) {
              const uint32_t c = (word >> (sh + i * vb)) & cmask;
              // Lloyd-Max values are summed in the rotated basis (rotated back after the merge)
              vh[e][i] = a.val_mode == 0 ? fmaf(v1, (float)c, v0) : v0 * s_vc[c];
            }
          }
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            if (h < G) {
              const float4 wq = *reinterpret_cast<const float4*>(&s_w[h * 64 + u0]);
#pragma unroll
              for (int i = 0; i < M; ++i) {
                float acc = o[h][i];
                acc = fmaf(wq.x, vh[0][i], acc);
                acc = fmaf(wq.y, vh[1][i], acc);
                acc = fmaf(wq.z, vh[2][i], acc);
                acc = fmaf(wq.w, vh[3][i], acc);
                o[h][i] = acc;
              }
            }
          }
        }
      }
    }
    gen_wave_sync();   // s_w and s_vs are rewritten by the next block
  }

  // merge the four waves, head by head, into the split's partial
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) continue;   // uniform over the work-group
    if (lane == 0) {
      s_part[wave * (2 + D)] = m_run[h];
      s_part[wave * (2 + D) + 1] = l_run[h];
    }
#pragma unroll
    for (int i = 0; i < M; ++i) s_part[wave * (2 + D) + 2 + lane * M + i] = o[h][i];
    __syncthreads();
    if (wave == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kGenWaves; ++w) mx = fmaxf(mx, s_part[w * (2 + D)]);
      float Ls = 0.f, O[M];
#pragma unroll
      for (int i = 0; i < M; ++i) O[i] = 0.f;
#pragma unroll
      for (int w = 0; w < kGenWaves; ++w) {
        const float* pw = s_part + w * (2 + D);
        const float f = pw[0] == -INFINITY ? 0.f : exp2f(pw[0] - mx);
        Ls = fmaf(f, pw[1], Ls);
#pragma unroll
        for (int i = 0; i < M; ++i) O[i] = fmaf(f, pw[2 + lane * M + i], O[i]);
      }
      float* dst = a.ws + ((((int64_t)b * a.hkv + kvh) * a.splits + split) * G + h) * (2 + D);
      if (lane == 0) {
        dst[0] = mx;
        dst[1] = Ls;
      }
#pragma unroll
      for (int i = 0; i < M; ++i) dst[2 + lane * M + i] = O[i];
    }
    __syncthreads();
  }
}

// Decode attention, merge part: one wave per (q head, sequence) combines the
// splits' partials by log-sum-exp and writes the output (Lloyd-Max values: rotated
// back, s * H o / sqrt(d)).  A sequence with no valid token gets zeros.
template <int D>
__global__ __launch_bounds__(64) void gen_merge_kernel(GenDecodeArgs a) {
  constexpr int M = D / 64;
  constexpr float isd = (float)inv_sqrt_dim<D>();
  const int qh = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int G = a.group, kvh = qh / G, h = qh - kvh * G;
  const int64_t stride = (int64_t)G * (2 + D);
  const float* src = a.ws + (((int64_t)b * a.hkv + kvh) * a.splits * G + h) * (2 + D);
  // lane s holds split s's max and sum (at most 64 splits), so they are read in one
  // round trip; each split's weight then reaches every lane from its own lane
  const int ns = a.splits;
  float ms = -INFINITY, ls = 0.f;
  if (lane < ns) {
    ms = src[lane * stride];
    ls = src[lane * stride + 1];
  }
  const float mx = gw_max(ms);
  const float fl = (ms == -INFINITY || mx == -INFINITY) ? 0.f : exp2f(ms - mx);
  const float L = gw_sum(fl * ls);
  float O[M];
#pragma unroll
  for (int i = 0; i < M; ++i) O[i] = 0.f;
  // the splits' rows, eight at a time with their loads in flight together
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float pv[8][M];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < M; ++i) pv[u][i] = s0 + u < ns ? src[(s0 + u) * stride + 2 + lane * M + i] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fl), min(s0 + u, 63)));
#pragma unroll
      for (int i = 0; i < M; ++i) O[i] = fmaf(f, pv[u][i], O[i]);
    }
  }
  float r[M];
#pragma unroll
  for (int i = 0; i < M; ++i) r[i] = L > 0.f ? O[i] / L : 0.f;
  if (a.val_mode == 1) {
    gen_fwht<M, float>(r, lane);
#pragma unroll
    for (int i = 0; i < M; ++i) r[i] *= a.c->signs[lane * M + i] * isd;
  }
  float* out = a.out + ((int64_t)b * a.hkv * G + qh) * D + lane * M;
#pragma unroll
  for (int i = 0; i < M; ++i) out[i] = r[i];
}

// ---------------------------------------------------------------------------
// Dequantize: one wave per (list entry, KV head): k_hat = norm * s * H C[code] /
// sqrt(d) (stage 1 for QJL keys); values min + scale * code (Lloyd-Max values as
// the keys).  A slot outside the cache gives a zero row; a row outside the buffer
// is skipped.
template <int D>
__global__ __launch_bounds__(64 * kGenWaves) void gen_dequant_kernel(GenDequantArgs a) {
  constexpr int M = D / 64;
  constexpr float isd = (float)inv_sqrt_dim<D>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float sg[M];
#pragma unroll
  for (int i = 0; i < M; ++i) sg[i] = a.c->signs[lane * M + i];
  const int64_t nvec = a.n * a.hkv;
  for (int64_t e = (int64_t)blockIdx.x * kGenWaves + wave; e < nvec; e += (int64_t)gridDim.x * kGenWaves) {
    const int64_t i_ent = e / a.hkv;
    const int h = (int)(e - i_ent * a.hkv);
    const int64_t row = a.rows ? a.rows[i_ent] : i_ent;
    if (row < 0 || row >= a.buf_rows) continue;
    const int64_t slot = a.slots[i_ent];
    float kx[M], vx[M];
#pragma unroll
    for (int i = 0; i < M; ++i) kx[i] = vx[i] = 0.f;
    if (slot >= 0 && slot < a.num_blocks * 16) {
      const uint8_t* page = a.cache + ((slot >> 4) * a.hkv + h) * (int64_t)a.f.page_bytes;
      const int so = (int)(slot & 15);
      const uint8_t* krow = page + a.f.kcodes + so * a.rows_b.kcodes;
#pragma unroll
      for (int i = 0; i < M; ++i) kx[i] = a.c->kc[gen_read_code(krow, 1, a.key_bits, lane * M + i)];
      if (a.key_mode != 3) {   // FP8 keys: the E4M3 values themselves
        const float norm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
        gen_fwht<M, float>(kx, lane);
#pragma unroll
        for (int i = 0; i < M; ++i) kx[i] *= sg[i] * isd * norm;
      }
      const uint8_t* vrow = page + a.f.vcodes + so;
      if (a.val_mode == 0) {
        const float mn = reinterpret_cast<const float*>(page + a.f.vmin)[so];
        const float sc = reinterpret_cast<const float*>(page + a.f.vscale)[so];
#pragma unroll
        for (int i = 0; i < M; ++i) vx[i] = fmaf(sc, (float)gen_read_code(vrow, 16, a.val_bits, lane * M + i), mn);
      } else {
        const float vn = reinterpret_cast<const float*>(page + a.f.vmin)[so];
#pragma unroll
        for (int i = 0; i < M; ++i) vx[i] = a.c->vc[gen_read_code(vrow, 16, a.val_bits, lane * M + i)];
        gen_fwht<M, float>(vx, lane);
#pragma unroll
        for (int i = 0; i < M; ++i) vx[i] *= sg[i] * isd * vn;
      }
    }
    const int64_t o = (row * a.hkv + h) * D + lane * M;
    if (a.bf16_out) {
      uint16_t* ko = static_cast<uint16_t*>(a.k_out) + o;
      uint16_t* vo = static_cast<uint16_t*>(a.v_out) + o;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        ko[i] = __builtin_bit_cast(uint16_t, (__bf16)kx[i]);
        vo[i] = __builtin_bit_cast(uint16_t, (__bf16)vx[i]);
      }
    } else {
      float* ko = static_cast<float*>(a.k_out) + o;
      float* vo = static_cast<float*>(a.v_out) + o;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        ko[i] = kx[i];
        vo[i] = vx[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_gen_append(const GenAppendArgs& a, int d, int grid, hipStream_t s) {
  const int64_t waves = a.num_tokens * a.hkv;
  if (waves <= 0) return hipSuccess;
  const dim3 g((unsigned)std::min<int64_t>((waves + kGenWaves - 1) / kGenWaves, std::max(1, grid)));
  switch (d) {
    case 64:
      if (a.bf16) hipLaunchKernelGGL((gen_append_kernel<64, true>), g, dim3(64 * kGenWaves), 0, s, a);
      else hipLaunchKernelGGL((gen_append_kernel<64, false>), g, dim3(64 * kGenWaves), 0, s, a);
      break;
    case 256:
      if (a.bf16) hipLaunchKernelGGL((gen_append_kernel<256, true>), g, dim3(64 * kGenWaves), 0, s, a);
      else hipLaunchKernelGGL((gen_append_kernel<256, false>), g, dim3(64 * kGenWaves), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int GM>
hipError_t gen_decode_dg(const GenDecodeArgs& a, hipStream_t s) {
  const dim3 g((unsigned)a.splits, (unsigned)a.hkv, (unsigned)a.batch);
  const size_t lds =
      (size_t)gen_decode_lds(D, a.group, a.key_mode == 2, (int)a.rows.vcodes, a.key_bits == 4 || a.key_bits == 2)
          .bytes;
  switch (a.key_bits) {
    case 2: hipLaunchKernelGGL((gen_decode_kernel<D, 2, GM>), g, dim3(64 * kGenWaves), lds, s, a); break;
    case 3: hipLaunchKernelGGL((gen_decode_kernel<D, 3, GM>), g, dim3(64 * kGenWaves), lds, s, a); break;
    case 4: hipLaunchKernelGGL((gen_decode_kernel<D, 4, GM>), g, dim3(64 * kGenWaves), lds, s, a); break;
    case 8: hipLaunchKernelGGL((gen_decode_kernel<D, 8, GM>), g, dim3(64 * kGenWaves), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t gen_decode_d(const GenDecodeArgs& a, hipStream_t s) {
  // register arrays sized for up to 4 or up to 16 query heads per KV head
  const hipError_t e = a.group <= 4 ? gen_decode_dg<D, 4>(a, s) : gen_decode_dg<D, kGenMaxGroup>(a, s);
  if (e != hipSuccess) return e;
  const dim3 gm((unsigned)(a.hkv * a.group), (unsigned)a.batch);
  hipLaunchKernelGGL(gen_merge_kernel<D>, gm, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gen_decode(const GenDecodeArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return gen_decode_d<64>(a, s);
    case 256: return gen_decode_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gen_dequant(const GenDequantArgs& a, int d, int grid, hipStream_t s) {
  const int64_t waves = a.n * a.hkv;
  if (waves <= 0) return hipSuccess;
  const dim3 g((unsigned)std::min<int64_t>((waves + kGenWaves - 1) / kGenWaves, std::max(1, grid)));
  switch (d) {
    case 64: hipLaunchKernelGGL(gen_dequant_kernel<64>, g, dim3(64 * kGenWaves), 0, s, a); break;
    case 256: hipLaunchKernelGGL(gen_dequant_kernel<256>, g, dim3(64 * kGenWaves), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
