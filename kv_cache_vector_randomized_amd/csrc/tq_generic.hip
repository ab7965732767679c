// Generic path for gfx950: head_dim 64, 128 or 256 and up to 16 query heads per
// KV head, for the configurations the tuned kernels do not take (head_dim other
// than 128, or a group size other than 1, 2 and 4).  Same page format and the
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

__device__ __forceinline__ float gw_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double gw_sum64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float gw_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float gw_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m));
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
      const T p = __shfl_xor(x[i], m);
      x[i] = upper ? p - x[i] : x[i] + p;
    }
  }
}

// This lane's coordinates of row `row` of a [rows][d] activation array (bf16 or fp32).
template <int M>
__device__ __forceinline__ void gen_load(const void* base, int64_t row, bool bf16, int lane, float (&x)[M]) {
  constexpr int D = 64 * M;
  if (bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row * D + lane * M;
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] = __uint_as_float((uint32_t)p[i] << 16);
  } else {
    const float* p = static_cast<const float*>(base) + row * D + lane * M;
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] = p[i];
  }
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
// Quantize-append: one wave per (token, KV head).  Keys: ||k|| and the rotation in
// fp64 (the squares of fp32 or bf16 values are exact there), codes of the unit
// coordinate, the stored norm (plain or corrected) rounded once to fp32, and for
// QJL keys the residual r = y - norm * C[code] in the rotated frame, its norm and
// the signs of S r (fp64 sums of fp32 S).  Values: uniform (min, scale =
// fl32((max - min) / (2^b - 1)), code = rint((v - min) / scale) with the quotient
// in fp64) or Lloyd-Max as the keys with a plain norm.
template <int D>
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

    // ---- keys
    float kf[M];
    gen_load<M>(a.k, vi, a.bf16 != 0, lane, kf);
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
      // rows lane*M + i of S r: 16 rows of S^T requested before they are used
      double pr[M];
#pragma unroll
      for (int i = 0; i < M; ++i) pr[i] = 0.0;
      for (int k0 = 0; k0 < D; k0 += 16) {
        float sv[16][M];
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
          for (int i = 0; i < M; ++i) sv[u][i] = a.St[(k0 + u) * D + lane * M + i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
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
    gen_wave_sync();   // every read of s_codes is done before the values overwrite it

    // ---- values
    float vf[M];
    gen_load<M>(a.v, vi, a.bf16 != 0, lane, vf);
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
      const double vn = sqrt(gw_sum64(vs));
      gen_fwht<M, double>(zv, lane);
      const double ivu = vn > 0.0 ? isd / vn : 0.0;
#pragma unroll
      for (int i = 0; i < M; ++i) s_codes[wave][lane * M + i] = (uint8_t)gen_code(s_vt, a.val_bits, zv[i] * ivu);
      if (lane == 0) reinterpret_cast<float*>(page + a.f.vmin)[so] = (float)vn;
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
// <coef S q'', 2 sigma - 1> for QJL keys).  Each wave keeps a running max, sum and
// weighted value sum per head; the work-group's four are merged through LDS and
// stored as the split's partial (max, sum, d sums) per head.
template <int D>
__global__ __launch_bounds__(64 * kGenWaves) void gen_decode_kernel(GenDecodeArgs a) {
  constexpr int M = D / 64;
  constexpr int GM = kGenMaxGroup;
  constexpr float isd = (float)inv_sqrt_dim<D>();
  __shared__ float s_q[GM][D];
  __shared__ float s_p[GM][D];
  __shared__ float s_kc[256], s_vc[16];
  __shared__ float s_w[kGenWaves][GM][64];
  __shared__ float s_part[kGenWaves][2 + D];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int hq = a.hkv * G;
  for (int i = tid; i < 256; i += 64 * kGenWaves) s_kc[i] = a.c->kc[i];
  if (tid < 16) s_vc[tid] = a.c->vc[tid];
  for (int h = wave; h < G; h += kGenWaves) {
    float x[M];
    gen_load<M>(a.q, (int64_t)b * hq + (int64_t)kvh * G + h, a.q_bf16 != 0, lane, x);
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] *= a.c->signs[lane * M + i];
    gen_fwht<M, float>(x, lane);
    const float f = a.scale * isd * kGenLog2e;
#pragma unroll
    for (int i = 0; i < M; ++i) s_q[h][lane * M + i] = x[i] * f;
  }
  __syncthreads();
  const bool qjl = a.key_mode == 2;
  if (qjl) {
    for (int h = wave; h < G; h += kGenWaves) {
      float acc[M];
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = 0.f;
      for (int k0 = 0; k0 < D; k0 += 16) {
        float sv[16][M];
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
          for (int i = 0; i < M; ++i) sv[u][i] = a.St[(k0 + u) * D + lane * M + i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float qk = s_q[h][k0 + u];
#pragma unroll
          for (int i = 0; i < M; ++i) acc[i] = fmaf(sv[u][i], qk, acc[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < M; ++i) s_p[h][lane * M + i] = acc[i] * a.qjl_coef;
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
    float lg[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) lg[h] = -INFINITY;
    if (valid) {
      const uint8_t* page = a.cache + ((int64_t)blk * a.hkv + kvh) * pstride;
      const float norm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
      const uint8_t* krow = page + a.f.kcodes + so * a.rows.kcodes;
      float dot[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) dot[h] = 0.f;
      for (int i = 0; i < D; ++i) {
        const float c = s_kc[gen_read_code(krow, 1, a.key_bits, i)];
#pragma unroll
        for (int h = 0; h < GM; ++h)
          if (h < G) dot[h] = fmaf(s_q[h][i], c, dot[h]);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) lg[h] = norm * dot[h];
      if (qjl) {
        const float rho = reinterpret_cast<const float*>(page + a.f.kres)[so];
        const uint8_t* srow = page + a.f.ksigns + so * a.rows.ksigns;
        float cs[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) cs[h] = 0.f;
        for (int j = 0; j < D; ++j) {
          const float sgn = ((srow[j >> 3] >> (j & 7)) & 1u) ? 1.f : -1.f;
#pragma unroll
          for (int h = 0; h < GM; ++h)
            if (h < G) cs[h] = fmaf(sgn, s_p[h][j], cs[h]);
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) lg[h] = fmaf(norm, dot[h], rho * cs[h]);
      }
      if (a.logits != nullptr) {
#pragma unroll
        for (int h = 0; h < GM; ++h)
          if (h < G) a.logits[((int64_t)b * hq + (int64_t)kvh * G + h) * a.max_seq + t] = lg[h] * kGenLn2;
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
        s_w[wave][h][lane] = p;
      }
    }
    gen_wave_sync();
    // values of the block's tokens: lane l adds coordinates l*M .. l*M + M - 1
    for (int u = 0; u < 64; ++u) {
      if (__shfl(valid ? 1 : 0, u) == 0) continue;   // uniform
      const int bu = __shfl(blk, u);
      const int su = (tb + u) & 15;
      const uint8_t* pg = a.cache + ((int64_t)bu * a.hkv + kvh) * pstride;
      const uint8_t* vrow = pg + a.f.vcodes + su;
      float vh[M];
      if (a.val_mode == 0) {
        const float mn = reinterpret_cast<const float*>(pg + a.f.vmin)[su];
        const float sc = reinterpret_cast<const float*>(pg + a.f.vscale)[su];
#pragma unroll
        for (int i = 0; i < M; ++i) vh[i] = fmaf(sc, (float)gen_read_code(vrow, 16, a.val_bits, lane * M + i), mn);
      } else {
        // Lloyd-Max values are summed in the rotated basis (rotated back after the merge)
        const float vn = reinterpret_cast<const float*>(pg + a.f.vmin)[su];
#pragma unroll
        for (int i = 0; i < M; ++i) vh[i] = vn * s_vc[gen_read_code(vrow, 16, a.val_bits, lane * M + i)];
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const float w = s_w[wave][h][u];
#pragma unroll
          for (int i = 0; i < M; ++i) o[h][i] = fmaf(w, vh[i], o[h][i]);
        }
      }
    }
    gen_wave_sync();   // s_w is rewritten by the next block
  }

  // merge the four waves, head by head, into the split's partial
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) continue;   // uniform over the work-group
    if (lane == 0) {
      s_part[wave][0] = m_run[h];
      s_part[wave][1] = l_run[h];
    }
#pragma unroll
    for (int i = 0; i < M; ++i) s_part[wave][2 + lane * M + i] = o[h][i];
    __syncthreads();
    if (wave == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kGenWaves; ++w) mx = fmaxf(mx, s_part[w][0]);
      float L = 0.f, O[M];
#pragma unroll
      for (int i = 0; i < M; ++i) O[i] = 0.f;
#pragma unroll
      for (int w = 0; w < kGenWaves; ++w) {
        const float mw = s_part[w][0];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - mx);
        L = fmaf(f, s_part[w][1], L);
#pragma unroll
        for (int i = 0; i < M; ++i) O[i] = fmaf(f, s_part[w][2 + lane * M + i], O[i]);
      }
      float* dst = a.ws + ((((int64_t)b * a.hkv + kvh) * a.splits + split) * G + h) * (2 + D);
      if (lane == 0) {
        dst[0] = mx;
        dst[1] = L;
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
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, src[s * stride]);
  float L = 0.f, O[M];
#pragma unroll
  for (int i = 0; i < M; ++i) O[i] = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float* p = src + s * stride;
      const float f = p[0] == -INFINITY ? 0.f : exp2f(p[0] - mx);
      L = fmaf(f, p[1], L);
#pragma unroll
      for (int i = 0; i < M; ++i) O[i] = fmaf(f, p[2 + lane * M + i], O[i]);
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
      const float norm = reinterpret_cast<const float*>(page + a.f.knorm)[so];
      const uint8_t* krow = page + a.f.kcodes + so * a.rows_b.kcodes;
#pragma unroll
      for (int i = 0; i < M; ++i) kx[i] = a.c->kc[gen_read_code(krow, 1, a.key_bits, lane * M + i)];
      gen_fwht<M, float>(kx, lane);
#pragma unroll
      for (int i = 0; i < M; ++i) kx[i] *= sg[i] * isd * norm;
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
    case 64: hipLaunchKernelGGL(gen_append_kernel<64>, g, dim3(64 * kGenWaves), 0, s, a); break;
    case 128: hipLaunchKernelGGL(gen_append_kernel<128>, g, dim3(64 * kGenWaves), 0, s, a); break;
    case 256: hipLaunchKernelGGL(gen_append_kernel<256>, g, dim3(64 * kGenWaves), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gen_decode(const GenDecodeArgs& a, int d, hipStream_t s) {
  const dim3 g((unsigned)a.splits, (unsigned)a.hkv, (unsigned)a.batch);
  const dim3 gm((unsigned)(a.hkv * a.group), (unsigned)a.batch);
  switch (d) {
    case 64:
      hipLaunchKernelGGL(gen_decode_kernel<64>, g, dim3(64 * kGenWaves), 0, s, a);
      hipLaunchKernelGGL(gen_merge_kernel<64>, gm, dim3(64), 0, s, a);
      break;
    case 128:
      hipLaunchKernelGGL(gen_decode_kernel<128>, g, dim3(64 * kGenWaves), 0, s, a);
      hipLaunchKernelGGL(gen_merge_kernel<128>, gm, dim3(64), 0, s, a);
      break;
    case 256:
      hipLaunchKernelGGL(gen_decode_kernel<256>, g, dim3(64 * kGenWaves), 0, s, a);
      hipLaunchKernelGGL(gen_merge_kernel<256>, gm, dim3(64), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gen_dequant(const GenDequantArgs& a, int d, int grid, hipStream_t s) {
  const int64_t waves = a.n * a.hkv;
  if (waves <= 0) return hipSuccess;
  const dim3 g((unsigned)std::min<int64_t>((waves + kGenWaves - 1) / kGenWaves, std::max(1, grid)));
  switch (d) {
    case 64: hipLaunchKernelGGL(gen_dequant_kernel<64>, g, dim3(64 * kGenWaves), 0, s, a); break;
    case 128: hipLaunchKernelGGL(gen_dequant_kernel<128>, g, dim3(64 * kGenWaves), 0, s, a); break;
    case 256: hipLaunchKernelGGL(gen_dequant_kernel<256>, g, dim3(64 * kGenWaves), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
