// Dequantize kernel for gfx950: stored codes back to vectors in the original
// basis (issoh.co.jp "TurboQuantとは？…", 第1段: the inverse of the random
// rotation is diag(s) H / sqrt(d); qiita AMD LMCache article: decoding is
// separate from byte transport, D(T(Q(X))) = D(Q(X))), written to caller-chosen
// rows of a running buffer (turboquant-vllm write-up, "Incremental
// dequantization": only the step's new tokens are reconstructed and appended).
//
// The kernel writes 4 (bf16) or 8 (fp32) times the bytes it reads, so it is
// bound by the stores and by VALU issue.  Work split: a wave takes 32
// consecutive list entries of one kv head, 8 at a time.  Eight lanes share a
// token: lane bits {0, 1, 3} give the lane's part p (0..7), lane bits {2, 4, 5}
// the token.  Part p holds the groups of G consecutive coordinates 8Gm + Gp + e
// (G = 4 for fp32 output, 8 for bf16; e < G, m < 16/G), so one store
// instruction writes a whole 128-byte line of each of 8 output rows.  The
// Hadamard butterfly runs over the 4 coordinate bits of e and m inside the lane
// and over the 3 bits of p with one DPP fused multiply-add per value (partners
// at lane distance 1, 2 and 8).
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kStageBytes = kMaxPageBytes;   // the largest page (FP8 keys, 4-bit uniform values)
constexpr int kStageLoads = (kStageBytes + 1023) / 1024;   // 16-byte loads per lane to stage a page
// groups of 16 list entries per wave (measured: one for fp32 output, two for bf16)
template <bool BF16OUT>
constexpr int groups_per_wave() { return BF16OUT ? 2 : 1; }

// Cross-lane butterfly stage: every lane computes x_own + x_partner * t, where t =
// +1 in the lower lane of the pair and -1 in the upper.  Values are held multiplied
// by a per-lane sign rho (start 1); with registers R = rho * x the same
// instruction, R_own + R_partner * t, leaves R' = rho * t * (x_partner + t * x_own),
// i.e. the butterfly output times the new sign rho * t, because partner lanes share
// every other lane bit and so share rho.  The signs are removed at the end.
// The s_nop covers the DPP read-after-VALU-write hazard of the first value.
#define TQ_FMAC16(CTL)                                                                               \
  asm volatile("s_nop 1\n\t"                                                                         \
               "v_fmac_f32_dpp %0, %0, %16 " CTL "\n\tv_fmac_f32_dpp %1, %1, %16 " CTL "\n\t"        \
               "v_fmac_f32_dpp %2, %2, %16 " CTL "\n\tv_fmac_f32_dpp %3, %3, %16 " CTL "\n\t"        \
               "v_fmac_f32_dpp %4, %4, %16 " CTL "\n\tv_fmac_f32_dpp %5, %5, %16 " CTL "\n\t"        \
               "v_fmac_f32_dpp %6, %6, %16 " CTL "\n\tv_fmac_f32_dpp %7, %7, %16 " CTL "\n\t"        \
               "v_fmac_f32_dpp %8, %8, %16 " CTL "\n\tv_fmac_f32_dpp %9, %9, %16 " CTL "\n\t"        \
               "v_fmac_f32_dpp %10, %10, %16 " CTL "\n\tv_fmac_f32_dpp %11, %11, %16 " CTL "\n\t"    \
               "v_fmac_f32_dpp %12, %12, %16 " CTL "\n\tv_fmac_f32_dpp %13, %13, %16 " CTL "\n\t"    \
               "v_fmac_f32_dpp %14, %14, %16 " CTL "\n\tv_fmac_f32_dpp %15, %15, %16 " CTL           \
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),  \
                 "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),           \
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15])                                                \
               : "v"(t))

__device__ __forceinline__ void xstage0(float (&x)[16], float t) {
  TQ_FMAC16("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf");
}
__device__ __forceinline__ void xstage1(float (&x)[16], float t) {
  TQ_FMAC16("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf");
}
__device__ __forceinline__ void xstage3(float (&x)[16], float t) {
  TQ_FMAC16("row_ror:8 row_mask:0xf bank_mask:0xf");
}
#undef TQ_FMAC16

// Unnormalized Sylvester transform of the 128 coordinates held by 8 lanes.  The
// lane's 16 values x[Gm + e] are coordinates 8Gm + Gp + e, so the four bits of the
// index of x are coordinate bits (butterflies inside the lane) and the three lane
// bits of p the remaining ones.  On return x holds rho times the result, rho =
// (-1)^(lane bit 0 + lane bit 1 + lane bit 3).
__device__ __forceinline__ void wht_part(float (&x)[16], int lane) {
#pragma unroll
  for (int len = 1; len < 16; len <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i += 2 * len) {
#pragma unroll
      for (int j = i; j < i + len; ++j) {
        const float u = x[j], w = x[j + len];
        x[j] = u + w;
        x[j + len] = u - w;
      }
    }
  }
  xstage0(x, (lane & 1) ? -1.f : 1.f);   // lane bit 0 (p bit 0)
  xstage1(x, (lane & 2) ? -1.f : 1.f);   // lane bit 1 (p bit 1)
  xstage3(x, (lane & 8) ? -1.f : 1.f);   // lane bit 3 (p bit 2)
}

// A group is the G codes of coordinates 8Gm + Gp .. +G-1: GB bits starting at
// stream bit B(8Gm + Gp), first code in the low bits.  Keys (slot-major rows) are
// read with one aligned load per group when the group is whole bytes (B = 2, 4),
// else byte by byte; values (plane-major: byte q of a slot at 16q) byte by byte.
template <int B, int G>
struct Group {
  static constexpr int kBit(int p, int m) { return B * (8 * G * m + G * p); }
  static constexpr bool kWide = B != 3;                  // aligned 1-, 2- or 4-byte word
  static constexpr int kBytes = B == 3 ? (G == 8 ? 3 : 2) : B * G / 8;
  static constexpr int kRawKey = B == 8 ? G / 4 : kWide ? 1 : kBytes;   // raw registers per key group
};

template <int B, int G>
__device__ __forceinline__ void load_key_group(const uint8_t* krow, int p, int m, uint32_t* raw) {
  constexpr int n = Group<B, G>::kBytes;
  const int q = Group<B, G>::kBit(p, m) >> 3;
  if constexpr (B == 8) {   // FP8 keys: G bytes, dword-aligned
#pragma unroll
    for (int i = 0; i < G / 4; ++i) raw[i] = reinterpret_cast<const uint32_t*>(krow + q)[i];
  } else if constexpr (Group<B, G>::kWide) {
    if constexpr (n == 4) raw[0] = *reinterpret_cast<const uint32_t*>(krow + q);
    else if constexpr (n == 2) raw[0] = *reinterpret_cast<const uint16_t*>(krow + q);
    else raw[0] = krow[q];
  } else {
#pragma unroll
    for (int j = 0; j < n; ++j) raw[j] = krow[q + j];
  }
}

template <int B, int G>
__device__ __forceinline__ void load_value_group(const uint8_t* vslot, int p, int m, uint32_t* raw) {
  const int q = Group<B, G>::kBit(p, m) >> 3;
#pragma unroll
  for (int j = 0; j < Group<B, G>::kBytes; ++j) raw[j] = vslot[16 * (q + j)];
}

// The group word from its raw bytes (or its one wide word).
template <int B, int G, bool WIDE>
__device__ __forceinline__ uint32_t group_word(const uint32_t* raw, int p, int m) {
  if constexpr (WIDE) return raw[0];
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < Group<B, G>::kBytes; ++j) w |= raw[j] << (8 * j);
  if constexpr (B * G == 32) return w;
  return (w >> (Group<B, G>::kBit(p, m) & 7)) & ((1u << (B * G)) - 1u);
}

// Codebook values of G codes through the LDS table built for B bits: pairs of
// 4-bit codes per byte, quads of 2-bit codes per byte, single 3-bit codes.
template <int B, int G>
__device__ __forceinline__ void table_lookup(const float* tbl, uint32_t w, float* y) {
  if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < G / 2; ++k) {
      const f32x2 a = reinterpret_cast<const f32x2*>(tbl)[(w >> (8 * k)) & 0xFFu];
      y[2 * k] = a.x; y[2 * k + 1] = a.y;
    }
  } else if constexpr (B == 2) {
#pragma unroll
    for (int k = 0; k < G / 4; ++k) {
      const floatx4 a = reinterpret_cast<const floatx4*>(tbl)[(w >> (8 * k)) & 0xFFu];
      y[4 * k] = a.x; y[4 * k + 1] = a.y; y[4 * k + 2] = a.z; y[4 * k + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < G; ++e) y[e] = tbl[(w >> (3 * e)) & 7u];
  }
}

// Table entries: B = 4: 256 float pairs; B = 2: 256 float quads; B = 3: 8 floats;
// B = 8: 256 floats (one code per byte, read straight from the raw words).
template <int B>
constexpr int table_floats() { return B == 8 ? 256 : B == 4 ? 512 : (B == 2 ? 1024 : 8); }

template <int B>
__device__ __forceinline__ void build_table(float* tbl, const float* c, int tid) {
  if constexpr (B == 8) {
    tbl[tid] = c[tid];   // 256 threads, one code each
  } else if constexpr (B == 4) {
    tbl[2 * tid] = c[tid & 15];
    tbl[2 * tid + 1] = c[tid >> 4];
  } else if constexpr (B == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) tbl[4 * tid + e] = c[(tid >> (2 * e)) & 3];
  } else {
    if (tid < 8) tbl[tid] = c[tid];
  }
}

// Stores of the lane's values: fp32 groups of 4 (16 bytes; 8 lanes write 128
// contiguous bytes), bf16 groups of 8 (16 bytes likewise), rounded to nearest even.
template <bool BF16OUT>
__device__ __forceinline__ void store_part(void* buf, int64_t elem, int p, const float (&x)[16]) {
  constexpr int G = BF16OUT ? 8 : 4;
#pragma unroll
  for (int m = 0; m < 16 / G; ++m) {
    const int c = 8 * G * m + G * p;
    const float* y = x + G * m;
    if constexpr (BF16OUT) {
      uint32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        u[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[2 * k], y[2 * k + 1]}, bf16x2));
      __builtin_nontemporal_store((u32x4){u[0], u[1], u[2], u[3]},
                                  reinterpret_cast<u32x4*>(static_cast<uint16_t*>(buf) + elem + c));
    } else {
      __builtin_nontemporal_store((floatx4){y[0], y[1], y[2], y[3]},
                                  reinterpret_cast<floatx4*>(static_cast<float*>(buf) + elem + c));
    }
  }
}

// x = scale * s (.) H C[code] for one Lloyd-Max row from its group words; sgn
// bit i = sign to apply to value i (the rotation's sign of its coordinate times rho).
__device__ __forceinline__ void rotate_scale(float (&x)[16], float scale, uint32_t sgn, int lane) {
  wht_part(x, lane);
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = __uint_as_float(__float_as_uint(x[e] * scale) ^ (((sgn >> e) & 1u) << 31));
}

template <int B, int G>
__device__ __forceinline__ void lloyd_part(const uint32_t* words, const float* tbl, float scale, uint32_t sgn,
                                           int lane, float (&x)[16]) {
#pragma unroll
  for (int m = 0; m < 16 / G; ++m) table_lookup<B, G>(tbl, words[m], x + G * m);
  rotate_scale(x, scale, sgn, lane);
}

// Raw fields of one list entry: key and value group bytes (or words) and scalars.
template <int KB, int VB, int G>
struct Raw {
  uint32_t k[16 / G][Group<KB, G>::kRawKey];
  uint32_t v[16 / G][Group<VB, G>::kBytes];
  float knrm, vmn, vsc;
};

// Read the fields of slot `so` of a page (in global memory or staged in LDS).
template <int KB, int VB, int G, bool VLM, bool FP8>
__device__ __forceinline__ void load_raw(const uint8_t* pg, const FieldOffsets& f, int so, int p,
                                         Raw<KB, VB, G>& r) {
#pragma unroll
  for (int m = 0; m < 16 / G; ++m) {
    load_key_group<KB, G>(pg + f.kcodes + so * (KB * 16), p, m, r.k[m]);
    load_value_group<VB, G>(pg + f.vcodes + so, p, m, r.v[m]);
  }
  r.knrm = FP8 ? 1.f : reinterpret_cast<const float*>(pg + f.knorm)[so];
  r.vmn = reinterpret_cast<const float*>(pg + f.vmin)[so];
  r.vsc = VLM ? 0.f : reinterpret_cast<const float*>(pg + f.vscale)[so];
}

// Reconstruct one entry from its raw fields (ok = 0 gives zeros) and store it to
// row rw when rw is inside the buffer.
template <int KB, int VB, int G, bool VLM, bool BF16OUT, bool FP8>
__device__ __forceinline__ void finish(const DequantArgs& a, const Raw<KB, VB, G>& r, bool ok, int64_t rw, uint32_t h,
                                       const float* ktbl, const float* vtbl, uint32_t sgn, int lane, int p) {
  uint32_t vw[16 / G];
#pragma unroll
  for (int m = 0; m < 16 / G; ++m) vw[m] = group_word<VB, G, false>(r.v[m], p, m);
  float xk[16], xv[16];
  if constexpr (FP8) {
    // FP8 keys: the E4M3 values themselves (exact conversions), no rotation
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int m = 0; m < 16 / G; ++m)
#pragma unroll
      for (int i = 0; i < G / 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(r.k[m][i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(r.k[m][i], true);
        float* y = xk + G * m + 4 * i;
        y[0] = ok ? lo.x : 0.f; y[1] = ok ? lo.y : 0.f; y[2] = ok ? hi.x : 0.f; y[3] = ok ? hi.y : 0.f;
      }
  } else if constexpr (KB == 8) {
    // 8-bit codes: one table read per byte of the raw words, then the rotation
#pragma unroll
    for (int m = 0; m < 16 / G; ++m)
#pragma unroll
      for (int i = 0; i < G / 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) xk[G * m + 4 * i + e] = ktbl[(r.k[m][i] >> (8 * e)) & 0xFFu];
    rotate_scale(xk, ok ? r.knrm * kInvSqrtDim : 0.f, sgn, lane);
  } else {
    uint32_t kw[16 / G];
#pragma unroll
    for (int m = 0; m < 16 / G; ++m) kw[m] = group_word<KB, G, Group<KB, G>::kWide>(r.k[m], p, m);
    lloyd_part<KB, G>(kw, ktbl, ok ? r.knrm * kInvSqrtDim : 0.f, sgn, lane, xk);
  }
  if constexpr (VLM) {
    lloyd_part<VB, G>(vw, vtbl, ok ? r.vmn * kInvSqrtDim : 0.f, sgn, lane, xv);
  } else {
    const float vsc = ok ? r.vsc : 0.f, vm = ok ? r.vmn : 0.f;
#pragma unroll
    for (int m = 0; m < 16 / G; ++m)
#pragma unroll
      for (int e = 0; e < G; ++e) xv[G * m + e] = fmaf(vsc, (float)((vw[m] >> (VB * e)) & ((1u << VB) - 1u)), vm);
  }
  if (rw >= 0 && rw < a.buf_rows) {
    const int64_t elem = (rw * a.hkv + h) * kDim;
    store_part<BF16OUT>(a.k_out, elem, p, xk);
    store_part<BF16OUT>(a.v_out, elem, p, xv);
  }
}

}  // namespace

// A wave's entries form kGroups groups of 16.  A group that is one whole page in
// slot order (the usual case when a whole sequence is reconstructed) is read
// with kStageLoads 16-byte loads per lane, all issued at the start, and staged
// in LDS; any other group is read entry by entry.
template <int KB, int VB, bool VLM, bool BF16OUT, bool FP8>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  __shared__ __align__(16) float ktbl[table_floats<KB>()];
  __shared__ __align__(16) float vtbl[VLM ? table_floats<VB>() : 1];
  constexpr int kGroups = groups_per_wave<BF16OUT>();
  __shared__ __align__(16) uint8_t stage[4][kGroups][kStageBytes];   // a page per group
  const int tid = threadIdx.x;
  if constexpr (!FP8) build_table<KB>(ktbl, a.c->kc, tid);
  if constexpr (VLM) build_table<VB>(vtbl, a.c->vc, tid);
  __syncthreads();
  constexpr int G = BF16OUT ? 8 : 4;   // consecutive coordinates per group
  const int lane = tid & 63;
  const int p = (lane & 3) | ((lane >> 1) & 4);          // part: lane bits 0, 1, 3
  const int t = ((lane >> 2) & 1) | ((lane >> 3) & 6);   // token: lane bits 2, 4, 5
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (chunk of 16 kGroups list entries, kv head) of this wave; the host keeps it below 2^32
  const uint32_t item = blockIdx.x * 4u + (uint32_t)wave;
  const uint32_t chunk = item / (uint32_t)a.hkv;
  const uint32_t h = item - chunk * (uint32_t)a.hkv;
  const int64_t first = (int64_t)chunk * (16 * kGroups);
  if (first >= a.n) return;   // uniform over the wave
  // per value Gm+e: the rotation's sign of coordinate 8Gm + Gp + e, times rho
  uint32_t sgn = 0;
#pragma unroll
  for (int m = 0; m < 16 / G; ++m) {
    const int c = 8 * G * m + G * p;
    sgn |= ((a.sign_bits[c >> 5] >> (c & 31)) & ((1u << G) - 1u)) << (G * m);
  }
  if (__popc(lane & 11) & 1) sgn ^= 0xFFFFu;
  const int64_t slot_end = a.num_blocks * kBlockTokensDev;
  const uint32_t pb = a.f.page_bytes;
  // Whole-page groups: slot of entry first + 16g + j in lane j (and j + 16, ...).
  bool whole[kGroups];
  const uint8_t* gpage[kGroups];
  u32x4 st[kGroups][kStageLoads];
  int64_t sl[kGroups], wrow[kGroups][2];
  bool in[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {   // both groups' slots and rows before any page load
    const int64_t ie = first + 16 * g + (lane & 15);
    in[g] = ie < a.n;
    sl[g] = a.slots[in[g] ? ie : a.n - 1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t i = first + 16 * g + 8 * j + t;
      const int64_t ic = i < a.n ? i : a.n - 1;
      wrow[g][j] = i < a.n ? (a.rows ? a.rows[ic] : ic) : -1;
    }
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int64_t s0 = ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)sl[g] >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sl[g]);
    const bool mine = in[g] && sl[g] == s0 + (lane & 15);
    whole[g] = __all(mine) && (s0 & 15) == 0 && s0 >= 0 && s0 < slot_end;
    const uint32_t pg = (uint32_t)(whole[g] ? s0 >> 4 : 0) * (uint32_t)a.hkv + h;
    gpage[g] = a.cache + (uint64_t)pg * pb;
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (whole[g]) {
#pragma unroll
      for (int k = 0; k < kStageLoads; ++k) {
        const uint32_t off = 16u * (lane + 64 * k);
        if (off < pb) st[g][k] = *reinterpret_cast<const u32x4*>(gpage[g] + off);
      }
    }
  }
  // stage every page before the first store, so that no wait for these loads
  // also waits for stores
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (whole[g]) {
#pragma unroll
      for (int k = 0; k < kStageLoads; ++k) {
        const uint32_t off = 16u * (lane + 64 * k);
        if (off < pb) *reinterpret_cast<u32x4*>(stage[wave][g] + off) = st[g][k];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int64_t e0 = first + 16 * g;
    if (e0 >= a.n) break;   // uniform
    if (whole[g]) {
      // the wave's own LDS writes complete before its later LDS reads
      const uint8_t* sp = stage[wave][g];
      Raw<KB, VB, G> r[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) load_raw<KB, VB, G, VLM, FP8>(sp, a.f, 8 * j + t, p, r[j]);
#pragma unroll
      for (int j = 0; j < 2; ++j) finish<KB, VB, G, VLM, BF16OUT, FP8>(a, r[j], true, wrow[g][j], h, ktbl, vtbl, sgn, lane, p);
    } else {
      Raw<KB, VB, G> r[2];
      bool ok[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t i = e0 + 8 * j + t;   // the same entry for the token's 8 lanes
        const bool ine = i < a.n;
        const int64_t slot = a.slots[ine ? i : a.n - 1];
        ok[j] = ine && slot >= 0 && slot < slot_end;
        // an entry without a valid slot reads the (in-bounds) constant block and is zeroed
        const uint32_t pg = (uint32_t)(slot >> 4) * (uint32_t)a.hkv + h;   // < 2^32 for any cache in memory
        const uint8_t* pgp = ok[j] ? a.cache + (uint64_t)pg * pb : reinterpret_cast<const uint8_t*>(a.c);
        load_raw<KB, VB, G, VLM, FP8>(pgp, a.f, ok[j] ? (int)(slot & 15) : 0, p, r[j]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) finish<KB, VB, G, VLM, BF16OUT, FP8>(a, r[j], ok[j], wrow[g][j], h, ktbl, vtbl, sgn, lane, p);
    }
  }
}

namespace {

static_assert(sizeof(DevConsts) >= kMaxPageBytes, "invalid slots read a page's worth of the constant block");

template <int KB, int VB, bool FP8>
hipError_t dequant_launch(const DequantArgs& a, bool lm, bool bf16, hipStream_t s) {
  const int per_wave = 16 * (bf16 ? groups_per_wave<true>() : groups_per_wave<false>());
  const int64_t items = (a.n + per_wave - 1) / per_wave * a.hkv;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (lm) {
    if constexpr (KB == 8) return hipErrorInvalidValue;   // 8-bit and FP8 keys pair with uniform values
    else if (bf16) hipLaunchKernelGGL((dequant_kernel<KB, VB, true, true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dequant_kernel<KB, VB, true, false, false>), grid, dim3(256), 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((dequant_kernel<KB, VB, false, true, FP8>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dequant_kernel<KB, VB, false, false, FP8>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int KB, bool FP8>
hipError_t dequant_vb(const DequantArgs& a, int val_bits, bool lm, bool bf16, hipStream_t s) {
  switch (val_bits) {
    case 2: return dequant_launch<KB, 2, FP8>(a, lm, bf16, s);
    case 3: return dequant_launch<KB, 3, FP8>(a, lm, bf16, s);
    case 4: return dequant_launch<KB, 4, FP8>(a, lm, bf16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, int key_bits, int key_mode, int val_bits, int val_mode, bool bf16_out,
                          hipStream_t s) {
  const bool lm = val_mode == TQ_VAL_LLOYD;
  if (key_mode == TQ_KEY_POLAR) return lm ? hipErrorInvalidValue : launch_polar_dequant(a, key_bits, val_bits, bf16_out, s);
  switch (key_bits) {
    case 8:
      return key_mode == TQ_KEY_FP8 ? dequant_vb<8, true>(a, val_bits, lm, bf16_out, s)
                                    : dequant_vb<8, false>(a, val_bits, lm, bf16_out, s);
    case 2: return dequant_vb<2, false>(a, val_bits, lm, bf16_out, s);
    case 3: return dequant_vb<3, false>(a, val_bits, lm, bf16_out, s);
    case 4: return dequant_vb<4, false>(a, val_bits, lm, bf16_out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
