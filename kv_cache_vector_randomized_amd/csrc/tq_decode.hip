// Decode attention over the packed cache for gfx950 (one launch, split merge included).
//
// Sources (page and section): issoh.co.jp "TurboQuantとは？…", the section on
// where the zero-loss claim comes from (logits against 4-bit keys are the part
// that is sped up); ai-navigate-news turboquant-vllm write-up (attention has to
// be fused over the compressed cache); lilting.ch TurboQuant article, QJL section
// (query kept in full precision, projected with the same S; corrected score).
//
// One work-group of 8 waves per (split of the context, kv head, sequence), one
// work-group per compute unit; the waves take the split's 64-token tiles (4 pages
// of 16 tokens) one at a time from a counter in LDS, so they finish together.
//
// Logits: per tile, rows = (query head, term of the query), columns = 16 tokens
// of one page, K = 32 coordinates, on the f16 16x16x32 MFMA.  The rotated query
// and the centroids are each split into f16 terms (query: three, codebook: two,
// both scaled by powers of two into f16's normal range), so the products carry
// about 22 significant bits; the fp32 accumulation keeps them.  Lane (j, g) of
// the B operand holds coordinates 32g..32g+31 of token j, one 16-byte load per
// page, and turns each byte of codes into the f16 centroid pair of both terms
// with one table read.  The MFMA output leaves head l/16 in the row of lanes l,
// so the running max, the sums and the output rows of a head stay in one row of
// 16 lanes.
//
// Values (uniform): sum_t p_t (min_t + scale_t * code_t).  The min part is a
// per-head scalar; the code part is an exact integer product on the int8 16x16x64
// MFMA: per tile the weights p_t * scale_t of each head go on a fixed-point grid
// tied to that head's largest weight in the tile, split into four 7-bit limbs
// (rows = head x limb, columns = coordinates, K = the tile's 64 tokens).  Value
// codes are plane-major in a page, so lane l loads the planes of coordinates
// 8j..8j+7 (j = l%16) of page l/16 with contiguous 16-byte loads.  Lloyd-Max
// values are accumulated on the fp32 4x4x1 MFMA in the rotated basis and rotated
// back once at the end.
//
// Per-split partials (max, sum, 128 outputs) go to the workspace; the last
// work-group of each (sequence, kv head) to finish, found with a self-resetting
// arrival counter, merges them by log-sum-exp and writes the output.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two adjacent floats (8-byte aligned) as one agent-scope access.
__device__ __forceinline__ void store_agent2(float* p, float x, float y) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                     (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Wave-wide max (prologue only): DPP within rows of 16 lanes, then the row
// broadcasts; rows outside ROW_MASK keep their own value, neutral for max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1, 0xF>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E, 0xF>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141, 0xF>(v));   // row_half_mirror
  v = fmaxf(v, dpp<0x140, 0xF>(v));   // row_mirror
  v = fmaxf(v, dpp<0x142, 0xA>(v));   // row_bcast:15
  v = fmaxf(v, dpp<0x143, 0xC>(v));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Reductions of two values within each row of 16 lanes: every lane of a row ends
// with its row's result.  Each step pairs a lane with one of the complementary
// group (quad swaps, half-row mirror, row mirror), so nothing is counted twice.
// The s_nop instructions cover the DPP read-after-VALU-write hazard.
#define TQ_ROW2(OP, CTL) OP " %0, %0, %0 " CTL "\n\t" OP " %1, %1, %1 " CTL "\n\ts_nop 0\n\t"
#define TQ_ROW2_ALL(OP)                                                     \
  "s_nop 1\n\t" TQ_ROW2(OP, "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf") \
      TQ_ROW2(OP, "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf")           \
          TQ_ROW2(OP, "row_half_mirror row_mask:0xf bank_mask:0xf")           \
              TQ_ROW2(OP, "row_mirror row_mask:0xf bank_mask:0xf")
__device__ __forceinline__ void row_max2(float& a, float& b) {
  asm volatile(TQ_ROW2_ALL("v_max_f32_dpp") : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void row_sum2(float& a, float& b) {
  asm volatile(TQ_ROW2_ALL("v_add_f32_dpp") : "+v"(a), "+v"(b));
}
#undef TQ_ROW2_ALL
#undef TQ_ROW2

// Byte BYTE of x shifted left by SH (the compiler folds the byte select into a
// sub-dword operand of the shift).
template <int SH, int BYTE>
__device__ __forceinline__ uint32_t byte_shl(uint32_t x) {
  return ((x >> (8 * BYTE)) & 0xFFu) << SH;
}

__device__ __forceinline__ uint32_t f16bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
// x = hi + lo (+ lo2) in f16, each term the rounding of what the previous left
__device__ __forceinline__ void split_f16(float x, float& hi, float& lo, float& lo2) {
  hi = (float)(_Float16)x;
  const float r = x - hi;
  lo = (float)(_Float16)r;
  lo2 = (float)(_Float16)(r - lo);
}

__device__ __forceinline__ floatx4 mfma_f16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Block ids of the 4 pages of one tile (wave-uniform; -1: absent or out of range).
struct TilePages {
  int b[4];
};

// Loads are unconditional: an absent page (block id -1) reads block 0 in its
// place and the lanes of absent pages and of tokens past the end are masked
// after the loads, which keeps the load path free of branches.  The caller
// guarantees num_blocks >= 1.
__device__ __forceinline__ int64_t page_offset(int blk, int kvh, int64_t blk_stride, int64_t head_stride) {
  return (int64_t)(blk >= 0 ? blk : 0) * blk_stride + kvh * head_stride;
}

// Key data of one tile for lane (j = lane%16, g = lane/16): for each page pg of
// the tile, bytes 4*KB*g .. 4*KB*g + 4*KB - 1 of token j's code row (coordinates
// 32g..32g+31) and token j's scalars.  Every load of one page is wave-uniform in
// its page, so the page address stays scalar.
template <int KB, bool QJL>
struct KeyTile {
  uint32_t kc[4][KB];
  uint32_t sg[4];      // QJL: dword g of token j's sign row (coordinates 32g..32g+31)
  float knorm[4], va[4], vb[4], kres[4];
};

template <int KB, bool QJL>
__device__ __forceinline__ void load_key_codes(KeyTile<KB, QJL>& r, const DecodeArgs& a, const TilePages& tp, int kvh,
                                               int lane, int64_t blk_stride, int64_t head_stride) {
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {
    const uint8_t* page = a.cache + page_offset(tp.b[pg], kvh, blk_stride, head_stride);
    const uint8_t* row = page + a.f.kcodes + j * (16 * KB) + g * (4 * KB);
    if constexpr (KB == 8) {   // 8-bit codes or FP8 keys: 32 bytes
      const uint4 u = reinterpret_cast<const uint4*>(row)[0], w = reinterpret_cast<const uint4*>(row)[1];
      r.kc[pg][0] = u.x; r.kc[pg][1] = u.y; r.kc[pg][2] = u.z; r.kc[pg][3] = u.w;
      r.kc[pg][4] = w.x; r.kc[pg][5] = w.y; r.kc[pg][6] = w.z; r.kc[pg][7] = w.w;
    } else if constexpr (KB == 4) {
      const uint4 u = *reinterpret_cast<const uint4*>(row);
      r.kc[pg][0] = u.x; r.kc[pg][1] = u.y; r.kc[pg][2] = u.z; r.kc[pg][3] = u.w;
    } else if constexpr (KB == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(row);
      r.kc[pg][0] = u.x; r.kc[pg][1] = u.y;
    } else {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(row);
      r.kc[pg][0] = w[0]; r.kc[pg][1] = w[1]; r.kc[pg][2] = w[2];
    }
    if constexpr (QJL) r.sg[pg] = reinterpret_cast<const uint32_t*>(page + a.f.ksigns + 16 * j)[g];
    else r.sg[pg] = 0u;
  }
}

template <int KB, bool QJL, bool VLM, bool FP8>
__device__ __forceinline__ void load_key_scalars(KeyTile<KB, QJL>& r, const DecodeArgs& a, const TilePages& tp,
                                                 int kvh, int lane, int64_t blk_stride, int64_t head_stride) {
  const int j = lane & 15;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {
    const uint8_t* page = a.cache + page_offset(tp.b[pg], kvh, blk_stride, head_stride);
    r.knorm[pg] = FP8 ? 1.f : reinterpret_cast<const float*>(page + a.f.knorm)[j];   // FP8: no norm
    r.va[pg] = reinterpret_cast<const float*>(page + a.f.vmin)[j];
    r.vb[pg] = VLM ? 0.f : reinterpret_cast<const float*>(page + a.f.vscale)[j];
    r.kres[pg] = QJL ? reinterpret_cast<const float*>(page + a.f.kres)[j] : 0.f;
  }
}

// Uniform values: lane l loads, from page l/16 of the tile, the byte planes of
// coordinates 8j..8j+7 (j = l%16): VB planes of 16 slots, contiguous in the page.
template <int VB>
__device__ __forceinline__ void load_value_group(uint4 (&vq)[VB], const DecodeArgs& a, int blk, int kvh, int lane,
                                                 int64_t blk_stride, int64_t head_stride) {
  const uint4* src = reinterpret_cast<const uint4*>(a.cache + page_offset(blk, kvh, blk_stride, head_stride) +
                                                    a.f.vcodes + 16 * VB * (lane & 15));
#pragma unroll
  for (int i = 0; i < VB; ++i) vq[i] = src[i];
}

// Centroid table of the key codes: for each byte of codes (KB = 4: two codes;
// KB = 3: a 6-bit pair; KB = 2: four codes), the f16 terms (hi, lo) of C * 2^s of
// each code in coordinate order, hi first.  Interleaving the terms along K lets
// one MFMA add both terms of the centroid: the query terms are duplicated to
// match (see qd below).
template <int KB, bool FP8>
struct KeyTable {
  static constexpr int kEntries = FP8 ? 1 : KB == 3 ? 64 : 256;   // FP8 keys need none
  static constexpr int kWords = FP8 || KB == 8 ? 1 : KB == 2 ? 4 : 2;
  static constexpr int kCodes = KB == 2 ? 4 : KB == 8 ? 1 : 2;     // codes per entry (per byte of codes)
};

// FP8 keys: B operand of the logits MFMA for coordinates 32g + 8*KAP .. +7 of this
// lane's chunk: the E4M3 bytes converted to f16 (every finite E4M3 value is an
// f16 normal number, so both conversions are exact).
template <int KAP>
__device__ __forceinline__ uint4 fp8_key_operand(const uint32_t (&kc)[8]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x = kc[2 * KAP + i];
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
    w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo.x, lo.y));
    w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi.x, hi.y));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// B operand of the logits MFMA for coordinates 32g + 4*KAP .. 32g + 4*KAP + 3 of
// this lane's chunk (K = coordinate x term, 8 halves).
template <int KB, int KAP>
__device__ __forceinline__ uint4 key_operand(const uint32_t (&kc)[KB], const uint32_t* tab) {
  const char* t = reinterpret_cast<const char*>(tab);
  if constexpr (KB == 8) {   // one code per byte, one word per code
    const uint32_t x = kc[KAP];
    return make_uint4(tab[x & 0xFFu], tab[(x >> 8) & 0xFFu], tab[(x >> 16) & 0xFFu], tab[x >> 24]);
  } else if constexpr (KB == 4) {
    const uint32_t x = kc[KAP >> 1];
    const uint2 e0 = *reinterpret_cast<const uint2*>(t + byte_shl<3, 2 * (KAP & 1)>(x));
    const uint2 e1 = *reinterpret_cast<const uint2*>(t + byte_shl<3, 2 * (KAP & 1) + 1>(x));
    return make_uint4(e0.x, e0.y, e1.x, e1.y);
  } else if constexpr (KB == 2) {
    return *reinterpret_cast<const uint4*>(t + byte_shl<4, KAP & 3>(kc[KAP >> 2]));
  } else {
    // 12 bits per group of 4 codes: bits 12*KAP .. 12*KAP + 11 of the chunk
    constexpr int bit = 12 * KAP, w = bit >> 5, sh = bit & 31;
    uint32_t v;
    if constexpr (sh + 12 <= 32) v = kc[w] >> sh;
    else v = __builtin_amdgcn_alignbit(kc[w + 1], kc[w], sh);
    const uint2 e0 = *reinterpret_cast<const uint2*>(t + ((v << 3) & 0x1F8u));
    const uint2 e1 = *reinterpret_cast<const uint2*>(t + ((v >> 3) & 0x1F8u));
    return make_uint4(e0.x, e0.y, e1.x, e1.y);
  }
}

// Value codes of coordinates 2*lane, 2*lane+1 for the four tokens of one 32-bit
// word of the lane's byte plane(s): returns (lo, hi) with one code per byte.
template <int VB>
__device__ __forceinline__ void value_nibbles(uint32_t x0, uint32_t x1, int sh, uint32_t& lo, uint32_t& hi) {
  if constexpr (VB == 4) {
    lo = x0 & 0x0F0F0F0Fu;
    hi = (x0 >> 4) & 0x0F0F0F0Fu;
  } else if constexpr (VB == 2) {
    const uint32_t f = (x0 >> sh) & 0x0F0F0F0Fu;
    lo = f & 0x03030303u;
    hi = (f >> 2) & 0x03030303u;
  } else {
    // 6-bit field per byte: bits [sh, 8) of plane p0 and [0, sh - 2) of plane p0 + 1
    const uint32_t m1 = (0xFFu >> sh) * 0x01010101u;
    const uint32_t m2 = ((0xFFu << (8 - sh)) & 0xFFu) * 0x01010101u;
    const uint32_t f = (((x0 >> sh) & m1) | ((x1 << (8 - sh)) & m2)) & 0x3F3F3F3Fu;
    lo = f & 0x07070707u;
    hi = (f >> 3) & 0x07070707u;
  }
}

// Lloyd-Max values: byte plane(s) of this lane's two coordinates for the tile's
// 4 pages (16 tokens per page, one coalesced 16-byte load per page and plane).
template <int VB>
__device__ __forceinline__ void load_value_planes(uint4 (&vp)[VB == 3 ? 8 : 4], const DecodeArgs& a,
                                                  const TilePages& tp, int kvh, int lane, int64_t blk_stride,
                                                  int64_t head_stride) {
  constexpr int VROW = kDim * VB / 8;
  const int p0 = (VB == 4) ? lane : (VB == 2) ? (lane >> 1) : ((6 * lane) >> 3);
  const int p1 = (6 * lane >> 3) + 1 < VROW ? (6 * lane >> 3) + 1 : VROW - 1;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {
    const uint8_t* vbase = a.cache + page_offset(tp.b[pg], kvh, blk_stride, head_stride) + a.f.vcodes;
    vp[pg] = *reinterpret_cast<const uint4*>(vbase + p0 * 16);
    if constexpr (VB == 3) vp[4 + pg] = *reinterpret_cast<const uint4*>(vbase + p1 * 16);
  }
}

// Value codes of this lane's page and coordinates 8j..8j+7 (j = lane % 16) as
// the B operand of the int8 MFMA for coordinate 8j + m: one code per byte, byte s
// of dword w is slot 4w + s of the page.  Codes are packed LSB-first, so within a
// byte plane the shifts and masks below act on four slots at once.
template <int VB, int M>
__device__ __forceinline__ intx4 value_codes(const uint4 (&vq)[VB]) {
  uint32_t r[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (VB == 4) {
      const uint32_t x = u4get(vq[M >> 1], w);
      r[w] = (M & 1) ? ((x >> 4) & 0x0F0F0F0Fu) : (x & 0x0F0F0F0Fu);
    } else if constexpr (VB == 2) {
      const uint32_t x = u4get(vq[M >> 2], w);
      r[w] = (x >> (2 * (M & 3))) & 0x03030303u;
    } else {
      // 8 codes of 3 bits span the three planes p0, p1, p2 of the group
      const uint32_t p0 = u4get(vq[0], w), p1 = u4get(vq[1], w), p2 = u4get(vq[2], w);
      if constexpr (M == 0) r[w] = p0 & 0x07070707u;
      else if constexpr (M == 1) r[w] = (p0 >> 3) & 0x07070707u;
      else if constexpr (M == 2) r[w] = ((p0 >> 6) & 0x03030303u) | ((p1 << 2) & 0x04040404u);
      else if constexpr (M == 3) r[w] = (p1 >> 1) & 0x07070707u;
      else if constexpr (M == 4) r[w] = (p1 >> 4) & 0x07070707u;
      else if constexpr (M == 5) r[w] = ((p1 >> 7) & 0x01010101u) | ((p2 << 1) & 0x06060606u);
      else if constexpr (M == 6) r[w] = (p2 >> 2) & 0x07070707u;
      else r[w] = (p2 >> 5) & 0x07070707u;
    }
  }
  return intx4{(int)r[0], (int)r[1], (int)r[2], (int)r[3]};
}

// Seven-bit limb `sh/7` of four weights, one per byte.
__device__ __forceinline__ int limb4(const uint4& x, uint32_t sh) {
  const uint32_t b0 = (x.x >> sh) & 0x7Fu, b1 = (x.y >> sh) & 0x7Fu;
  const uint32_t b2 = (x.z >> sh) & 0x7Fu, b3 = (x.w >> sh) & 0x7Fu;
  return (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Bits 0..15 of e to the even and of o to the odd bit positions of a word.
__device__ __forceinline__ uint32_t interleave16(uint32_t e, uint32_t o) {
  auto spread = [](uint32_t x) {
    x &= 0xFFFFu;
    x = (x | (x << 8)) & 0x00FF00FFu;
    x = (x | (x << 4)) & 0x0F0F0F0Fu;
    x = (x | (x << 2)) & 0x33333333u;
    return (x | (x << 1)) & 0x55555555u;
  };
  return spread(e) | (spread(o) << 1);
}

// Fused append (one wave): quantize the new token (lane l holds its coordinates
// 2l, 2l+1 of the key k0, k1 and the value v0, v1) as the append kernels do (rotation, codes through the key grid, fp32 norm with the
// optional correction, QJL signs and residual norm, uniform values) and write its
// fields into slot `so` of `page`.  Lane l works on coordinates 2l, 2l+1 and
// returns their key centroids (c0, c1), the stored norm, the QJL residual norm and
// the signs (+1/-1) of rows 2l, 2l+1 of S r'; the dequantized value row goes to
// vhat.  codes / rbuf are LDS scratch of the wave.
template <int KB, bool QJL, int VB, bool FP8, bool POLAR>
__device__ void new_token_quantize(const DecodeArgs& a, float k0, float k1, float v0, float v1, int lane,
                                   uint8_t* page, bool st, int so, uint8_t (&codes)[2][kDim], float* vhat,
                                   float* rbuf,
                                   float& c0, float& c1, float& nhat, float& rho, float& sgn0, float& sgn1) {
  rho = 0.f;
  sgn0 = sgn1 = 1.f;
  int kc0 = 0, kc1 = 0;
  if constexpr (FP8) {
    // FP8 keys: the E4M3 bytes of the coordinates, their values for the logit
    const uint32_t b0 = fp8_e4m3(k0), b1 = fp8_e4m3(k1);
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 cv = __builtin_amdgcn_cvt_pk_f32_fp8(b0 | (b1 << 8), false);
    c0 = cv.x;
    c1 = cv.y;
    nhat = 1.f;
    if (st) *reinterpret_cast<uint16_t*>(page + a.f.kcodes + so * kDim + 2 * lane) = (uint16_t)(b0 | (b1 << 8));
  } else {
  // ||k|| of the stored norm in fp64 from the inputs (squares exact, one rounding to fp32 at the end)
  const double nk64 = sqrt(wave_sum64(fma((double)k0, (double)k0, (double)k1 * (double)k1)));
  // keys: z = H(s * k), then codes of u = z / ||z||
  float x0 = k0 * a.c->signs[2 * lane], x1 = k1 * a.c->signs[2 * lane + 1];
  {
    const float s0 = x0 + x1, d0 = x0 - x1;
    x0 = s0;
    x1 = d0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float p0 = __shfl_xor(x0, m), p1 = __shfl_xor(x1, m);
    const bool upper = (lane & m) != 0;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
  if constexpr (POLAR) {
    // PolarQuant: the tree over y = z / sqrt(d) across the wave as in the append
    // (node n of level L in lane n 2^(L-1)), each angle's cell index at its slot;
    // the root radius is the norm.  For the logit: the unit leaves of this lane's
    // coordinates, products of the cell centres' cos / sin along the path, top down.
    const float y0 = x0 * kInvSqrtDim, y1 = x1 * kInvSqrtDim;
    if (lane == 0) codes[0][kDim - 1] = 0;                   // the unused slot
    codes[0][polar_slot(1, lane)] = (uint8_t)polar_code<KB>(atan2f(y1, y0), true);
    float rad = sqrtf(fmaf(y0, y0, y1 * y1));
#pragma unroll
    for (int lv = 2; lv <= 7; ++lv) {
      const float u = rad, v = __shfl_xor(rad, 1 << (lv - 2));
      if ((lane & ((1 << (lv - 1)) - 1)) == 0)
        codes[0][polar_slot(lv, lane >> (lv - 1))] = (uint8_t)polar_code<KB>(atan2f(v, u), false);
      rad = sqrtf(fmaf(u, u, v * v));
    }
    nhat = (float)nk64;                                      // the root radius ||y|| = ||k||
    wave_sync_lds();
    float pf = 1.f;
#pragma unroll
    for (int lv = 7; lv >= 2; --lv) {
      const uint32_t cd = codes[0][polar_slot(lv, lane >> (lv - 1))];
      pf *= ((lane >> (lv - 2)) & 1) ? a.c->pcsU[2 * cd + 1] : a.c->pcsU[2 * cd];
    }
    const uint32_t c1d = codes[0][polar_slot(1, lane)];
    c0 = pf * a.c->pcs1[2 * c1d];
    c1 = pf * a.c->pcs1[2 * c1d + 1];
  } else {
  const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;     // a zero key gives codes 2^(b-1)
  if constexpr (KB == 8) {
    kc0 = code_bsearch8(a.c->kt, a.c->kc, x0 * inv, c0);
    kc1 = code_bsearch8(a.c->kt, a.c->kc, x1 * inv, c1);
  } else {
    kc0 = lut_code(a.c->klut, x0 * inv, a.klut_scale, a.klut_bias, c0);
    kc1 = lut_code(a.c->klut, x1 * inv, a.klut_scale, a.klut_bias, c1);
  }
  const float nk = (float)nk64;                            // ||k||
  const double c2 = wave_sum64(fma((double)c0, (double)c0, (double)c1 * (double)c1));
  nhat = stored_norm(nk64, c2, !QJL && a.key_nc);
  if constexpr (QJL) {
    // residual in the rotated frame r' = H(s*k)/sqrt(d) - ||k|| C[code], and S r'
    const float r0 = fmaf(-nk, c0, x0 * kInvSqrtDim), r1 = fmaf(-nk, c1, x1 * kInvSqrtDim);
    rho = sqrtf(wave_sum(fmaf(r0, r0, r1 * r1)));
    rbuf[2 * lane] = r0;
    rbuf[2 * lane + 1] = r1;
    wave_sync_lds();
    // 32 rows of S^T requested at a time, then used (a sched barrier keeps the
    // compiler from sinking each load to its use: one round trip per 32 rows
    // instead of one per 8)
    float p0 = 0.f, p1 = 0.f;
    for (int kb = 0; kb < kDim; kb += 32) {
      float2 sv[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) sv[u] = *reinterpret_cast<const float2*>(&a.c->St[(kb + u) * kDim + 2 * lane]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        p0 = fmaf(sv[u].x, rbuf[kb + u], p0);
        p1 = fmaf(sv[u].y, rbuf[kb + u], p1);
      }
    }
    sgn0 = p0 >= 0.f ? 1.f : -1.f;
    sgn1 = p1 >= 0.f ? 1.f : -1.f;
    const uint64_t em = __ballot(p0 >= 0.f), om = __ballot(p1 >= 0.f);
    if (st && lane < 4)
      reinterpret_cast<uint32_t*>(page + a.f.ksigns + 16 * so)[lane] =
          interleave16((uint32_t)(em >> (16 * lane)), (uint32_t)(om >> (16 * lane)));
  }
  }
  }
  // uniform values, as the append kernel: codes rint(fl32(x - mn) * (1 / sc)), ties to even
  const float mn = -wave_max(-fminf(v0, v1));
  const float mx = wave_max(fmaxf(v0, v1));
  constexpr float levels = (float)((1 << VB) - 1);
  const float sc = (mx - mn) / levels;
  const float vinv = sc > 0.f ? 1.f / sc : 0.f;
  const uint32_t vc0 = (uint32_t)rintf((v0 - mn) * vinv), vc1 = (uint32_t)rintf((v1 - mn) * vinv);
  vhat[2 * lane] = fmaf(sc, (float)vc0, mn);
  vhat[2 * lane + 1] = fmaf(sc, (float)vc1, mn);
  if constexpr (!POLAR) {
    codes[0][2 * lane] = (uint8_t)kc0;
    codes[0][2 * lane + 1] = (uint8_t)kc1;
  }
  codes[1][2 * lane] = (uint8_t)vc0;
  codes[1][2 * lane + 1] = (uint8_t)vc1;
  wave_sync_lds();
  if constexpr (KB == 8) {
    // 8-bit codes (and FP8 above): one byte per coordinate, the lane's two bytes
    if (st && !FP8) *reinterpret_cast<uint16_t*>(page + a.f.kcodes + so * kDim + 2 * lane) = (uint16_t)(kc0 | (kc1 << 8));
  } else if (st && lane < 16 * KB) {
    page[a.f.kcodes + so * 16 * KB + lane] = (uint8_t)stream_byte<KB>(codes[0], lane);
  }
  if (st && lane < 16 * VB) page[a.f.vcodes + 16 * lane + so] = (uint8_t)stream_byte<VB>(codes[1], lane);
  if (st && lane == 0) {
    if (!FP8) reinterpret_cast<float*>(page + a.f.knorm)[so] = nhat;
    reinterpret_cast<float*>(page + a.f.vmin)[so] = mn;
    reinterpret_cast<float*>(page + a.f.vscale)[so] = sc;
    if constexpr (QJL) reinterpret_cast<float*>(page + a.f.kres)[so] = rho;
  }
}

// Key formats of the kernel (template parameter KM).
constexpr int kKmLloyd = 0;   // Lloyd-Max codes with a stored norm (plain or corrected)
constexpr int kKmQjl = 1;     // Lloyd-Max codes + QJL residual signs and norm
constexpr int kKmFp8 = 2;     // E4M3 bytes of the raw key (KB = 8)
constexpr int kKmPolar = 3;   // PolarQuant angle codes (subtree-major) and the radius

// PolarQuant keys: the 32 coordinates 32g..32g+31 of one token (g = lane / 16) as
// unit-radius leaf factors times 2^14, rebuilt top down from the quarter's angle
// codes (slots 0..30 of the lane's chunk), the root angle and the quarter's
// level-6 angle.  tu: (cos, sin) of the higher levels' cell centres; jt: for a
// level-2 code c2 and a level-1 code c1, 2^14 cos(c2) (cos, sin)(c1) at [16 c2 + c1]
// and 2^14 sin(c2) (cos, sin)(c1) at 256 + 16 c2 + c1, so each level-2 node's four
// leaves take two reads and four products.  (All tables in LDS.)
template <int KB>
__device__ __forceinline__ void polar_leaves(const uint32_t (&kc)[KB], uint32_t root, uint32_t l6, int g,
                                             const float2* tu, const float2* jt, float (&f)[32]) {
  const float2 r7 = tu[root], r6 = tu[l6];
  float v[8];
  v[0] = ((g >> 1) ? r7.y : r7.x) * ((g & 1) ? r6.y : r6.x);
  // levels 5, 4, 3: 1, 2, 4 angles at slots 30, 28, 24
#pragma unroll
  for (int lv = 5, n = 1, base = 30; lv >= 3; --lv, n <<= 1, base -= n) {   // bases 30, 28, 24
#pragma unroll
    for (int i = n - 1; i >= 0; --i) {
      const float2 cs = tu[get_code<KB>(kc, base + i)];
      const float r = v[i];
      v[2 * i] = r * cs.x;
      v[2 * i + 1] = r * cs.y;
    }
  }
  // levels 2 (slots 16..23) and 1 (slots 0..15) together
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c2 = get_code<KB>(kc, 16 + i) << 4;
    const float2 ea = jt[c2 | get_code<KB>(kc, 2 * i)];
    const float2 eb = jt[256 + (c2 | get_code<KB>(kc, 2 * i + 1))];
    const float r = v[i];
    f[4 * i] = r * ea.x;
    f[4 * i + 1] = r * ea.y;
    f[4 * i + 2] = r * eb.x;
    f[4 * i + 3] = r * eb.y;
  }
}

template <int KB, int KM, int VB, bool VLM>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
  constexpr bool QJL = KM == kKmQjl;
  constexpr bool FP8 = KM == kKmFp8;   // FP8 keys: no rotation, no codebook, no norm
  constexpr bool POLAR = KM == kKmPolar;   // PolarQuant keys: leaf factors from the angles, radius as norm
  __shared__ float2 ptab[POLAR ? 16 : 1];  // (cos, sin) per code of levels 3..7
  __shared__ float2 pjt[POLAR ? 512 : 1];  // levels 2 and 1 jointly, times 2^14 (see polar_leaves)
  // head group hg = query heads 4*sub .. 4*sub + G - 1 (sub = hg % hsub) of KV head hg / hsub
  int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  if (a.hsub > 1 && a.xcd_pairs) {
    // The head groups of one (split, KV head, sequence) read the same pages: give
    // them linear ids 8 apart, which the dispatcher sends to the same XCD (its own
    // L2) one after the other.  Linear id f = 8q + r: head group q % hsub of unit
    // 8 (q / hsub) + r, units in the grid's own order (split, KV head, sequence).
    // The launcher sets xcd_pairs only when 8 * hsub divides the grid size.
    const uint32_t f = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t q = f >> 3, u = (q / (uint32_t)a.hsub) * 8u + (f & 7u);
    const uint32_t t = u / gridDim.x;
    split = (int)(u - t * gridDim.x);
    b = (int)(t / (uint32_t)a.hkv);
    hg = (int)(t - (uint32_t)b * a.hkv) * a.hsub + (int)(q % (uint32_t)a.hsub);
  }
  const int kvh = hg / a.hsub;
  const int ngrp = a.hkv * a.hsub;
  const int sub = hg - kvh * a.hsub;
  const int64_t qh0 = (int64_t)kvh * a.group + 4 * sub;   // first query head of the work-group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, grp = lane >> 4;   // column (token of a page) and row group (head) of the lane

  using Tab = KeyTable<KB, FP8>;
  // Shared by the 4 waves: the f16 terms of the rotated query rows ([head][term]
  // [coordinate], each half duplicated into both halves of a word to meet the
  // two centroid terms; the 4th term is zero) and of their QJL projections
  // ([head][term][coordinate pair]), the key centroid table, the sign table, the
  // fp32 query rows (QJL only) and the Lloyd-Max value codebook.
  __shared__ __align__(16) uint32_t qd[4][4][132];
  __shared__ __align__(16) uint32_t pt[QJL ? 4 : 1][4][68];
  __shared__ __align__(16) uint32_t ktab[Tab::kEntries * Tab::kWords];
  __shared__ __align__(16) uint4 stab[QJL ? 256 : 1];
  __shared__ __align__(16) float q_sh[QJL ? 4 : 1][kDim + 4];
  __shared__ float vcb[16];
  __shared__ int qexp[4], pexp[4];
  // per wave and head, the 64 tokens' value weights: fp32 (Lloyd-Max values) or
  // the fixed-point integers fed to the int8 MFMA (uniform values)
  __shared__ __align__(16) uint32_t wT[kDecodeWaves][4][68];
  __shared__ float part_ml[kDecodeWaves][4][2];
  __shared__ __align__(16) float part_o[kDecodeWaves][4][kDim];

  // Block ids of the work-group's pages ([tile - tile_begin][page]; -1: absent):
  // tiles are handed to the waves one at a time, so every wave may need any of them.
  __shared__ int blk_lds[kMaxPagesPerSplit];
  __shared__ unsigned tile_ctr;
  // Fused append: fp32 rotated query rows and QJL projections of the heads, the
  // new token's codes, dequantized value row and QJL residual.
  __shared__ __align__(16) float qf[VLM ? 1 : 4][kDim];
  __shared__ __align__(16) float pf[QJL ? 4 : 1][kDim];
  __shared__ __align__(16) uint8_t nt_codes[VLM ? 1 : 2][kDim];
  __shared__ __align__(16) float nt_vhat[VLM ? 1 : kDim];
  __shared__ __align__(16) float nt_r[QJL ? kDim : 1];

  const int G = min(4, a.group - 4 * sub);   // query heads of this work-group (1..4)
  // Split `split` owns tiles [tile_begin, tile_end): an even share of the longest
  // sequence's tiles (at most 64).
  const int tile_begin = (int)((uint32_t)(split * a.tiles_total) / (uint32_t)a.splits);
  const int tile_end = (int)((uint32_t)((split + 1) * a.tiles_total) / (uint32_t)a.splits);
  const int64_t head_stride = a.f.page_bytes;
  const int64_t blk_stride = head_stride * a.hkv;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  uint32_t (&wt)[4][68] = wT[wave];

  // ---- Prologue.  First the block ids of the wave's first tile (tile_begin +
  // wave) and of the range, the constants the shared tables need, the query row
  // of head `wave`, the sequence length and the block-table entry of its last
  // position (uniform: scalar loads), then the first tile's pages.
  // Only the first tile's ids are waited for before the pages are requested:
  // pages are read at every in-range block id, and which tokens count is decided
  // once the length (and the new token's block) is known.  So the first pages
  // are in flight after one round trip, and their latency overlaps the rest of
  // the prologue: the tables, the query rotation and the barrier.
  // (a table row with no entries is never read: seq_lens stands in for it)
  const int32_t* trow = a.max_blocks > 0 ? table : a.seq_lens + b;
  const int tmax = max(a.max_blocks - 1, 0);
  // Loads of the prologue are unconditional (heads >= G read head 0 and are
  // zeroed, a wave without a tile reads an in-range page): conditional loads
  // would make the compiler wait for every earlier load before the first use of
  // any.  The vector loads that one wait covers are issued in the order needed.
  int t_cur = tile_begin + wave;
  const int page_first = 4 * t_cur + (lane & 3);
  const int raw_first = trow[min(page_first, tmax)];
  const int e_st = min(tid, kMaxPagesPerSplit - 1);
  const int page_st = 4 * tile_begin + e_st;
  const int raw_st = trow[min(page_st, tmax)];
  const float kc_top = (FP8 || POLAR) ? 1.f : a.c->kc[(1 << KB) - 1];
  float kc_e[Tab::kCodes];
  if constexpr (!FP8 && !POLAR) {
    const int ent = tid & (Tab::kEntries - 1);
#pragma unroll
    for (int i = 0; i < Tab::kCodes; ++i) kc_e[i] = a.c->kc[(ent >> (KB * i)) & ((1 << KB) - 1)];
  }
  // The query pair of this lane (coordinates 2*lane, 2*lane+1) is one word in
  // bf16 or two in fp32; both words are always read (the second re-reads the
  // first for bf16) so that no branch separates the load from its use.
  uint32_t qw0, qw1;
  {
    const bool f32 = a.q_dtype != TQ_BF16;
    const int64_t qo = ((int64_t)b * a.hq + qh0 + (wave < G ? wave : 0)) * kDim + 2 * lane;
    const uint32_t* qp = f32 ? reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.q) + qo)
                             : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + qo);
    qw0 = qp[0];
    qw1 = qp[f32 ? 1 : 0];
  }
  const float sg0 = a.c->signs[2 * lane], sg1 = a.c->signs[2 * lane + 1];
  int seq_len = a.seq_lens[b];
  seq_len = max(0, min(seq_len, min(a.max_seq, 16 * a.max_blocks)));
  if (a.num_blocks <= 0) seq_len = 0;     // no page exists: every block id is absent
  const int last_raw = trow[min(max(seq_len - 1, 0) >> 4, tmax)];
  // keep the range's block ids here, read in the first tile ids' round trip:
  // left to the scheduler, the read sinks to its use behind the page loads,
  // and waiting for it there would wait for the pages too
  int raw_stv = raw_st;
  asm volatile("" : "+v"(raw_stv));
  // the first tile's block ids as read: loads go to in-range ids (block 0 stands
  // in for the others), validity is applied below
  TilePages tl;
  int vblk;            // block of the page this lane reads value planes from (page lane/16)
  {
    const int l = (page_first >= a.max_blocks || raw_first < 0 || (int64_t)raw_first >= a.num_blocks) ? -1 : raw_first;
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) tl.b[pg] = __builtin_amdgcn_readlane(l, pg);
    // (selects, not an LDS exchange: its wait would also cover the scalar loads in flight)
    vblk = grp == 0 ? tl.b[0] : grp == 1 ? tl.b[1] : grp == 2 ? tl.b[2] : tl.b[3];
  }

  KeyTile<KB, QJL> nx;
  uint4 vp[VB == 3 ? 8 : 4];     // Lloyd-Max values: byte planes of coordinates 2*lane, 2*lane+1
  uint4 vq[VB];                  // uniform values: the planes of coordinates 8j..8j+7 of page lane/16
  load_key_codes<KB, QJL>(nx, a, tl, kvh, lane, blk_stride, head_stride);
  load_key_scalars<KB, QJL, VLM, FP8>(nx, a, tl, kvh, lane, blk_stride, head_stride);
  if constexpr (VLM) load_value_planes<VB>(vp, a, tl, kvh, lane, blk_stride, head_stride);
  else load_value_group<VB>(vq, a, vblk, kvh, lane, blk_stride, head_stride);

  // Fused append: position seq_len - 1 is the new token (when its block exists); it
  // is left out of the tiles and enters through the work-group whose split holds it.
  const int new_blk = (!VLM && a.k_new != nullptr && seq_len > 0 && a.max_blocks > 0 && last_raw >= 0 &&
                       (int64_t)last_raw < a.num_blocks) ? last_raw : -1;
  const bool has_new = new_blk >= 0;
  const bool own_new = has_new && ((seq_len - 1) >> 6) >= tile_begin && ((seq_len - 1) >> 6) < tile_end;
  const int tok_end = min(seq_len - (has_new ? 1 : 0), tile_end * 64);
  // block ids of the range's pages (-1: absent or past the context), and of the
  // first tile's, with the same rule
  // (threads past the last entry store the same value to it: no branch for the
  // compiler to sink the read into, behind the page loads)
  blk_lds[e_st] = (e_st >= 4 * (tile_end - tile_begin) || page_st >= a.max_blocks || raw_stv < 0 ||
                   (int64_t)raw_stv >= a.num_blocks || page_st * 16 >= tok_end)
                      ? -1 : raw_stv;
  if (tid == 0) tile_ctr = kDecodeWaves;   // the first kDecodeWaves tiles go to the waves in order
  bool have = t_cur < tile_end && t_cur * 64 < tok_end;
  TilePages tp;
  {
    const int v = (!have || page_first >= a.max_blocks || raw_first < 0 || (int64_t)raw_first >= a.num_blocks ||
                   page_first * 16 >= tok_end)
                      ? -1 : raw_first;
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) tp.b[pg] = __builtin_amdgcn_readlane(v, pg);
  }

  // Key centroid table: C * 2^s2 with 2^s2 bringing the largest |C| (the last,
  // the codebook being symmetric) into [2^14, 2^15).
  // (PolarQuant: leaf factors are in [-1, 1], scaled by 2^14)
  const int s2 = FP8 ? 0 : POLAR ? 14 : 15 - __builtin_amdgcn_frexp_expf(kc_top);
  if constexpr (POLAR) {
    // (the joint table also carries the 2^14 scale of the MFMA operand, so the leaves come out scaled)
    if (tid < 16) ptab[tid] = make_float2(a.c->pcsU[2 * tid], a.c->pcsU[2 * tid + 1]);
    if (tid < 512) {
      const int c2 = (tid >> 4) & 15, c1 = tid & 15;
      const float h = 16384.f * a.c->pcsU[2 * c2 + (tid >> 8)];   // cos (first child) or sin (second)
      pjt[tid] = make_float2(h * a.c->pcs1[2 * c1], h * a.c->pcs1[2 * c1 + 1]);
    }
  }
  if (!FP8 && !POLAR && tid < Tab::kEntries) {
    uint32_t* e = &ktab[tid * Tab::kWords];
#pragma unroll
    for (int i = 0; i < Tab::kCodes; ++i) {
      float hi, lo, unused;
      split_f16(ldexpf(kc_e[i], s2), hi, lo, unused);
      e[i] = f16bits(hi) | (f16bits(lo) << 16);
    }
  }
  if constexpr (QJL) {
    // bit e of a sign byte -> f16 +1 (bit set) or -1, for the 8 coordinates of the byte
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = ((tid >> (2 * i)) & 1 ? 0x3C00u : 0xBC00u) | (((tid >> (2 * i + 1)) & 1 ? 0x3C00u : 0xBC00u) << 16);
    if (tid < 256) stab[tid] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (VLM && tid < 16) vcb[tid] = a.c->vc[tid];

  // Rotate query head `wave` (waves 0..3): q'' = log2(e) * scale * H(s*q)/sqrt(d),
  // so that the logits come out in base-2 units for exp2.  Heads >= G stay zero.
  if (wave < kMaxGroup) {
    const bool f32 = a.q_dtype != TQ_BF16;
    float qx0 = f32 ? __uint_as_float(qw0) : bf16lo(qw0);
    float qx1 = f32 ? __uint_as_float(qw1) : bf16hi(qw0);
    if (wave >= G) qx0 = qx1 = 0.f;
    float x0 = qx0, x1 = qx1;
    if constexpr (!FP8) {
      x0 *= sg0;
      x1 *= sg1;
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
    }
    const float f = a.scale * (FP8 ? 1.f : kInvSqrtDim) * kLog2e;
    x0 *= f;
    x1 *= f;
    // f16 terms of q'' * 2^s1, 2^s1 bringing the head's largest |q''| into [2^14, 2^15)
    const float qm = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const int s1 = qm > 0.f ? 15 - __builtin_amdgcn_frexp_expf(qm) : 0;
    float h0, l0, m0, h1, l1, m1;
    split_f16(ldexpf(x0, s1), h0, l0, m0);
    split_f16(ldexpf(x1, s1), h1, l1, m1);
    if constexpr (FP8) {
      // FP8 keys take one f16 term each: the query terms are not duplicated
      qd[wave][0][lane] = f16bits(h0) | (f16bits(h1) << 16);
      qd[wave][1][lane] = f16bits(l0) | (f16bits(l1) << 16);
      qd[wave][2][lane] = f16bits(m0) | (f16bits(m1) << 16);
      qd[wave][3][lane] = 0u;
    } else {
      *reinterpret_cast<uint2*>(&qd[wave][0][2 * lane]) = make_uint2(f16bits(h0) * 0x10001u, f16bits(h1) * 0x10001u);
      *reinterpret_cast<uint2*>(&qd[wave][1][2 * lane]) = make_uint2(f16bits(l0) * 0x10001u, f16bits(l1) * 0x10001u);
      *reinterpret_cast<uint2*>(&qd[wave][2][2 * lane]) = make_uint2(f16bits(m0) * 0x10001u, f16bits(m1) * 0x10001u);
      *reinterpret_cast<uint2*>(&qd[wave][3][2 * lane]) = make_uint2(0u, 0u);
    }
    if (lane == 0) qexp[wave] = s1;
    if constexpr (!VLM) *reinterpret_cast<float2*>(&qf[wave][2 * lane]) = make_float2(x0, x1);
    if constexpr (QJL) {
      // p'' = coef * S q''  (coef = sqrt(pi/2)/m): lane computes rows 2*lane, 2*lane+1
      q_sh[wave][2 * lane] = x0;
      q_sh[wave][2 * lane + 1] = x1;
      wave_sync_lds();
      // (32 rows of S^T requested at a time, as in the new token's projection)
      float acc0 = 0.f, acc1 = 0.f;
      for (int kb = 0; kb < kDim; kb += 32) {
        float2 sv[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) sv[u] = *reinterpret_cast<const float2*>(&a.c->St[(kb + u) * kDim + 2 * lane]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const float qk = q_sh[wave][kb + u];
          acc0 = fmaf(sv[u].x, qk, acc0);
          acc1 = fmaf(sv[u].y, qk, acc1);
        }
      }
      acc0 *= a.qjl_coef;
      acc1 *= a.qjl_coef;
      *reinterpret_cast<float2*>(&pf[wave][2 * lane]) = make_float2(acc0, acc1);
      const float pm = wave_max(fmaxf(fabsf(acc0), fabsf(acc1)));
      const int sp = pm > 0.f ? 15 - __builtin_amdgcn_frexp_expf(pm) : 0;
      split_f16(ldexpf(acc0, sp), h0, l0, m0);
      split_f16(ldexpf(acc1, sp), h1, l1, m1);
      pt[wave][0][lane] = f16bits(h0) | (f16bits(h1) << 16);
      pt[wave][1][lane] = f16bits(l0) | (f16bits(l1) << 16);
      pt[wave][2][lane] = f16bits(m0) | (f16bits(m1) << 16);
      pt[wave][3][lane] = 0u;
      if (lane == 0) pexp[wave] = sp;
    }
  }
  // Fused append: the new token's key and value pairs of this lane, loaded before
  // the barrier as raw words (bf16: one word, fp32: two; the second re-reads the
  // first for bf16) and converted only where wave kMaxGroup quantizes them after
  // it.  A use here would wait for every earlier load, this wave's first tile
  // included, and hold the barrier for the whole work-group.
  uint32_t nt_kw0 = 0u, nt_kw1 = 0u, nt_vw0 = 0u, nt_vw1 = 0u;
  if constexpr (!VLM) {
    if (own_new && wave == kMaxGroup) {
      const bool f32 = a.q_dtype != TQ_BF16;
      const int64_t e0 = ((int64_t)b * a.hkv + kvh) * kDim + 2 * lane;
      const uint32_t* kp = f32 ? reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.k_new) + e0)
                               : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k_new) + e0);
      const uint32_t* vp = f32 ? reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.v_new) + e0)
                               : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v_new) + e0);
      nt_kw0 = kp[0];
      nt_kw1 = kp[f32 ? 1 : 0];
      nt_vw0 = vp[0];
      nt_vw1 = vp[f32 ? 1 : 0];
    }
  }
  __syncthreads();

  // A operands of the logits MFMA: row lane%16 = (head (lane/4)%4, term lane%4),
  // coordinates 32g + 4*kap + (0..3), each twice (g = lane/16).
  const uint32_t* qa_src = &qd[(lane >> 2) & 3][lane & 3][(FP8 ? 16 : 32) * grp];
  // base-2 logit of head grp = D * 2^-(s1 + s2) * norm (and the QJL part: D2 * 2^-sp * residual norm)
  const float lscale = ldexpf(1.f, -(qexp[grp] + s2));
  const float pscale = QJL ? ldexpf(1.f, -pexp[grp]) : 0.f;
  const uint32_t* ktab_p = ktab;

  // Running max (base 2) and partial sums of head grp over this lane's tokens.
  float m_run = -INFINITY, l_lane = 0.f, s_lane = 0.f;
  // Uniform values: lane l accumulates head l/16, coordinates 8(l%16) + m.
  float O[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) O[m] = 0.f;
  // Lloyd-Max values: rows = heads, columns = coordinates 2*lane, 2*lane+1.
  floatx4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = O0, O2 = O0, O3 = O0;
  const int vsh = (VB == 2) ? 4 * (lane & 1) : (VB == 3) ? ((6 * lane) & 7) : 0;
  if constexpr (!VLM) {
    if (own_new && wave == kMaxGroup) {
      const bool f32 = a.q_dtype != TQ_BF16;
      const float nt_k0 = f32 ? __uint_as_float(nt_kw0) : bf16lo(nt_kw0);
      const float nt_k1 = f32 ? __uint_as_float(nt_kw1) : bf16hi(nt_kw0);
      const float nt_v0 = f32 ? __uint_as_float(nt_vw0) : bf16lo(nt_vw0);
      const float nt_v1 = f32 ? __uint_as_float(nt_vw1) : bf16hi(nt_vw0);
      float nt_c0, nt_c1, nt_nhat, nt_rho, nt_s0, nt_s1;
      uint8_t* page = const_cast<uint8_t*>(a.cache) + (int64_t)new_blk * blk_stride + kvh * head_stride;
      new_token_quantize<KB, QJL, VB, FP8, POLAR>(a, nt_k0, nt_k1, nt_v0, nt_v1, lane, page, sub == 0,
                                                  (seq_len - 1) & 15, nt_codes,
                                      nt_vhat, nt_r, nt_c0, nt_c1, nt_nhat, nt_rho, nt_s0, nt_s1);
      // the new token's base-2 logit for each head, then the wave's softmax state
      // starts from it (weight 1 at its own max)
      float ell[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        ell[h] = wave_sum(fmaf(qf[h][2 * lane], nt_c0, qf[h][2 * lane + 1] * nt_c1)) * nt_nhat;
        if constexpr (QJL) ell[h] = fmaf(wave_sum(fmaf(pf[h][2 * lane], nt_s0, pf[h][2 * lane + 1] * nt_s1)), nt_rho, ell[h]);
      }
      const float my = grp == 0 ? ell[0] : grp == 1 ? ell[1] : grp == 2 ? ell[2] : ell[3];
      if (grp < G) {
        m_run = my;
        l_lane = j16 == 0 ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) O[m] = nt_vhat[8 * j16 + m];
      }
      if (a.logits != nullptr && lane < G) {
        const float mine = lane == 0 ? ell[0] : lane == 1 ? ell[1] : lane == 2 ? ell[2] : ell[3];
        a.logits[((int64_t)b * a.hq + qh0 + lane) * a.max_seq + seq_len - 1] = mine * kLn2;
      }
    }
  }

  while (have) {
    // The next tile of the work-group's range for this wave (handed out in order).
    unsigned got = 0;
    if (lane == 0) got = atomicAdd(&tile_ctr, 1u);
    const int t_nx = tile_begin + (int)__builtin_amdgcn_readfirstlane(got);
    const bool has_next = t_nx < tile_end && t_nx * 64 < tok_end;
    // Without a next tile the loads below re-read the current pages (cache hits,
    // results unused): unconditional loads keep the compiler's waits exact.
    TilePages tpn = tp;
    int nvblk = vblk;
    if (has_next) {
      const int* nb = &blk_lds[4 * (t_nx - tile_begin)];
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) tpn.b[pg] = __builtin_amdgcn_readfirstlane(nb[pg]);
      nvblk = nb[grp];
    }
    const int tile = t_cur;
    const KeyTile<KB, QJL> cur = nx;

    // Logits of head grp for tokens 16*pg + j16 of the tile's 4 pages.
    floatx4 D[4], D2[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      D[pg] = floatx4{0.f, 0.f, 0.f, 0.f};
      D2[pg] = D[pg];
    }
#define TQ_KAP(KAP)                                                         \
  {                                                                         \
    const uint4 qa = *reinterpret_cast<const uint4*>(qa_src + 4 * (KAP));  \
    _Pragma("unroll") for (int pg = 0; pg < 4; ++pg)                        \
        D[pg] = mfma_f16(qa, key_operand<KB, KAP>(cur.kc[pg], ktab_p), D[pg]); \
  }
    if constexpr (FP8) {
#pragma unroll
      for (int kap = 0; kap < 4; ++kap) {
        const uint4 qa = *reinterpret_cast<const uint4*>(qa_src + 4 * kap);
#pragma unroll
        for (int pg = 0; pg < 4; ++pg) {
          const uint4 kb = kap == 0 ? fp8_key_operand<0>(cur.kc[pg]) : kap == 1 ? fp8_key_operand<1>(cur.kc[pg])
                         : kap == 2 ? fp8_key_operand<2>(cur.kc[pg]) : fp8_key_operand<3>(cur.kc[pg]);
          D[pg] = mfma_f16(qa, kb, D[pg]);
        }
      }
    } else if constexpr (POLAR) {
      // slot 31 of each quarter: the root (quarter 0) and the level-6 angles (quarters 1, 2)
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
        const uint32_t c31 = cur.kc[pg][KB - 1] >> (32 - KB);
        const uint32_t root = (uint32_t)__shfl((int)c31, j16);
        const uint32_t l6 = (uint32_t)__shfl((int)c31, j16 + 16 * (1 + (grp >> 1)));
        float f[32];
        polar_leaves<KB>(cur.kc[pg], root, l6, grp, ptab, pjt, f);
#pragma unroll
        for (int kap = 0; kap < 8; ++kap) {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // x = hi + lo: hi keeps x's top 11 significant bits (an f16 value for
            // |x| >= 2^-14), lo = x - hi exactly, both packed toward zero in one
            // instruction (lo loses at most 2^-10 of itself: |error| < 2^-20 |x|)
            const float x = f[4 * kap + e];
            const float hi = __uint_as_float(__float_as_uint(x) & 0xFFFFE000u);
            wv[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi, x - hi));
          }
          const uint4 qa = *reinterpret_cast<const uint4*>(qa_src + 4 * kap);
          D[pg] = mfma_f16(qa, make_uint4(wv[0], wv[1], wv[2], wv[3]), D[pg]);
        }
      }
    } else {
      TQ_KAP(0) TQ_KAP(1) TQ_KAP(2) TQ_KAP(3) TQ_KAP(4) TQ_KAP(5) TQ_KAP(6) TQ_KAP(7)
    }
#undef TQ_KAP
    if constexpr (QJL) {
#pragma unroll
      for (int kap = 0; kap < 4; ++kap) {
        const uint4 pa = *reinterpret_cast<const uint4*>(&pt[(lane >> 2) & 3][lane & 3][16 * grp + 4 * kap]);
#pragma unroll
        for (int pg = 0; pg < 4; ++pg) {
          const uint4 sb = stab[(cur.sg[pg] >> (8 * kap)) & 0xFFu];
          D2[pg] = mfma_f16(pa, sb, D2[pg]);
        }
      }
    }
    // The key chunks are consumed: fetch the next tile's while this one finishes
    // (its scalars follow once this tile's are used).
    load_key_codes<KB, QJL>(nx, a, tpn, kvh, lane, blk_stride, head_stride);

    float lg[4], va[4], vb[4];
    bool valid[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      valid[pg] = tile * 64 + 16 * pg + j16 < tok_end && tp.b[pg] >= 0;
      float v = (D[pg][0] + D[pg][1] + D[pg][2]) * (lscale * cur.knorm[pg]);
      if (QJL) v = fmaf((D2[pg][0] + D2[pg][1] + D2[pg][2]) * pscale, cur.kres[pg], v);
      lg[pg] = valid[pg] ? v : -INFINITY;
      // masked lanes may have read another page: their scalars must not reach a sum
      va[pg] = valid[pg] ? cur.va[pg] : 0.f;
      vb[pg] = valid[pg] ? cur.vb[pg] : 0.f;
    }
    if (a.logits != nullptr && grp < G) {
      float* lrow = a.logits + ((int64_t)b * a.hq + qh0 + grp) * a.max_seq + tile * 64 + j16;
#pragma unroll
      for (int pg = 0; pg < 4; ++pg)
        if (valid[pg]) lrow[16 * pg] = lg[pg] * kLn2;
    }
    // Online softmax (base 2) of head grp: the row of 16 lanes shares the max;
    // the accumulators are rescaled only when some head's max moved.
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    float smax = fmaxf(fmaxf(vb[0], vb[1]), fmaxf(vb[2], vb[3]));   // largest value scale of the tile
    row_max2(mt, smax);
    const float mnew = fmaxf(m_run, mt);
    if (__builtin_amdgcn_read_exec() & __ballot(mnew != m_run)) {
      const float al = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
      l_lane *= al;
      s_lane *= al;
      m_run = mnew;
      if constexpr (VLM) {
        float ah[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) ah[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16 * h));
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          O0[h] *= ah[h];
          O1[h] *= ah[h];
          O2[h] *= ah[h];
          O3[h] *= ah[h];
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) O[m] *= al;
      }
    }
    const float ms = (m_run == -INFINITY) ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      pr[pg] = __builtin_amdgcn_exp2f(lg[pg] - ms);    // 0 for masked tokens
      l_lane += pr[pg];
      if (!VLM) s_lane = fmaf(pr[pg], va[pg], s_lane);
    }
    load_key_scalars<KB, QJL, VLM, FP8>(nx, a, tpn, kvh, lane, blk_stride, head_stride);
    if constexpr (VLM) {
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) wt[grp][16 * pg + j16] = __float_as_uint(pr[pg] * va[pg]);
      wave_sync_lds();
      // Values: rows = 4 heads, columns = coordinates 2*lane / 2*lane+1, one token per
      // MFMA; even and odd tokens go to separate accumulators.
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int tt = pg * 16 + 4 * kk;
          const uint4 wu = *reinterpret_cast<const uint4*>(&wt[lane & 3][tt]);
          const float4 w4 = make_float4(__uint_as_float(wu.x), __uint_as_float(wu.y), __uint_as_float(wu.z),
                                        __uint_as_float(wu.w));
          uint32_t lo, hi;
          uint32_t x1 = 0u;
          if constexpr (VB == 3) x1 = u4get(vp[4 + pg], kk);
          value_nibbles<VB>(u4get(vp[pg], kk), x1, vsh, lo, hi);
          float b0[4], b1[4];
          b0[0] = vcb[lo & 0xFF]; b0[1] = vcb[(lo >> 8) & 0xFF]; b0[2] = vcb[(lo >> 16) & 0xFF]; b0[3] = vcb[lo >> 24];
          b1[0] = vcb[hi & 0xFF]; b1[1] = vcb[(hi >> 8) & 0xFF]; b1[2] = vcb[(hi >> 16) & 0xFF]; b1[3] = vcb[hi >> 24];
          O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.x, b0[0], O0, 0, 0, 0);
          O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.x, b1[0], O1, 0, 0, 0);
          O2 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.y, b0[1], O2, 0, 0, 0);
          O3 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.y, b1[1], O3, 0, 0, 0);
          O0 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.z, b0[2], O0, 0, 0, 0);
          O1 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.z, b1[2], O1, 0, 0, 0);
          O2 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.w, b0[3], O2, 0, 0, 0);
          O3 = __builtin_amdgcn_mfma_f32_4x4x1f32(w4.w, b1[3], O3, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep one page's operands live at a time
      }
      load_value_planes<VB>(vp, a, tpn, kvh, lane, blk_stride, head_stride);
    } else {
      // Fixed-point weights of head grp on the grid 2^(E-27), 2^E just above the
      // bound pmax * smax of the tile's weights p_t * scale_t (pmax = exp2(mt - ms),
      // the weight of the tile's largest logit; every weight is below 2^27 units,
      // four 7-bit limbs).  Rounding costs at most half a unit per token, so the
      // error of a tile's sum is below 64 (2^b - 1) 2^-27 pmax smax, and the
      // tiles' pmax add up to at most the softmax denominator: the error of the
      // normalised output stays below (2^b - 1) 2^-21 times the largest scale,
      // at any context length.  (The rows of the MFMA are per head, so each head
      // takes its own grid.)
      const float pmax = __builtin_amdgcn_exp2f(mt - ms);
      const int E = __builtin_amdgcn_frexp_expf(pmax * smax);
#pragma unroll
      for (int pg = 0; pg < 4; ++pg)
        wt[grp][16 * pg + j16] = (uint32_t)fmaf(pr[pg], ldexpf(vb[pg], 27 - E), 0.5f);   // round to nearest
      wave_sync_lds();
      // A operand: row lane%16 = (head (lane/4)%4, limb lane%4), tokens 16g..16g+15
      // of page g = lane/16, one per byte.
      const uint4* wsrc = reinterpret_cast<const uint4*>(&wt[(lane >> 2) & 3][16 * grp]);
      const uint32_t lsh = 7u * (uint32_t)(lane & 3);
      const intx4 A = {limb4(wsrc[0], lsh), limb4(wsrc[1], lsh), limb4(wsrc[2], lsh), limb4(wsrc[3], lsh)};
      const float bsc = ldexpf(1.f, E - 27);
      const intx4 zero = {0, 0, 0, 0};
#define TQ_PV(M)                                                                                   \
      {                                                                                            \
        const intx4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, value_codes<VB, M>(vq), zero, 0, 0, 0); \
        const uint32_t u = (uint32_t)d[0] + ((uint32_t)d[1] << 7) + ((uint32_t)d[2] << 14);        \
        O[M] = fmaf(fmaf((float)d[3], 2097152.f, (float)u), bsc, O[M]);                             \
      }
      TQ_PV(0) TQ_PV(1) TQ_PV(2) TQ_PV(3) TQ_PV(4) TQ_PV(5) TQ_PV(6) TQ_PV(7)
#undef TQ_PV
      load_value_group<VB>(vq, a, nvblk, kvh, lane, blk_stride, head_stride);
    }
    wave_sync_lds();
    t_cur = t_nx;
    tp = tpn;
    vblk = nvblk;
    have = has_next;
  }

  // ---- Per-wave totals of head grp (every lane of the row), then merge the
  // waves of the work-group.
  row_sum2(l_lane, s_lane);
  if (j16 == 0) {
    part_ml[wave][grp][0] = m_run;
    part_ml[wave][grp][1] = l_lane;
  }
  if constexpr (VLM) {
    O0 += O2;
    O1 += O3;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      part_o[wave][h][2 * lane] = O0[h];
      part_o[wave][h][2 * lane + 1] = O1[h];
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(&part_o[wave][grp][8 * j16]);
    dst[0] = make_float4(O[0] + s_lane, O[1] + s_lane, O[2] + s_lane, O[3] + s_lane);
    dst[1] = make_float4(O[4] + s_lane, O[5] + s_lane, O[6] + s_lane, O[7] + s_lane);
  }
  __syncthreads();
  // Merge the waves: thread (head h = wave < G, coordinates 2*lane, 2*lane+1).
  const int h = wave;
  float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
  if (h < G) {
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, part_ml[w][h][0]);
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = part_ml[w][h][0];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = fmaf(f, part_ml[w][h][1], L);
      o0 = fmaf(f, part_o[w][h][2 * lane], o0);
      o1 = fmaf(f, part_o[w][h][2 * lane + 1], o1);
    }
  }
  if (a.splits > 1) {
    // Publish this split's partial; the last work-group of the (sequence, kv head)
    // to arrive merges all splits (log-sum-exp) and writes the output.  Partials
    // are written and read with agent-scope (device-coherent) accesses, so no
    // cache-wide write-back or invalidate is needed around the arrival counter.
    if (h < G) {
      float* dst = a.ws + ((((int64_t)b * ngrp + hg) * a.splits + split) * 4 + h) * (2 + kDim);
      // (records of 2 + 128 floats: every pair below is 8-byte aligned)
      if (lane == 0) store_agent2(dst, M, L);
      store_agent2(dst + 2 + 2 * lane, o0, o1);
    }
    // Ordering without cache-wide fences.  The partials above are agent-scope atomic
    // stores, so they are performed at the device's coherence point (not held in this
    // XCD's L2), and s_waitcnt(0) returns only once every one of them has completed
    // there.  The barrier then orders all threads' completed stores before the arrival
    // increment, an atomic performed at the same coherence point.  The work-group that
    // reads splits - 1 was therefore the last to arrive: every other work-group's
    // stores had completed before its increment, and the loads below are agent-scope
    // atomic loads, served by the coherence point, issued only after the increment
    // returned.  (A release increment and an acquire fence would write back and
    // invalidate the whole L2 of each XCD: measured 45.7 against 33.5 us per step.)
    __builtin_amdgcn_s_waitcnt(0);            // every store of this thread has completed
    __syncthreads();
    __shared__ int last;
    if (tid == 0) {
      // wraps back to 0 after `splits` arrivals, so the counter is left zero
      const unsigned prev = __builtin_amdgcn_atomic_inc32(a.counters + (int64_t)b * ngrp + hg,
                                                         (unsigned)(a.splits - 1), __ATOMIC_RELAXED, "agent");
      last = prev == (unsigned)(a.splits - 1);
    }
    __syncthreads();
    if (!last) return;
    // Every wave merges: head wave % 4 over the splits of parity wave / 4, 16 of
    // them per round trip (all their loads in flight together), then the two
    // parities combine through LDS.
    const int mh = wave & 3, par = wave >> 2;
    M = -INFINITY;
    L = o0 = o1 = 0.f;
    if (mh < G) {
      const int64_t stride = 4 * (2 + kDim);
      const float* src = a.ws + (((int64_t)b * ngrp + hg) * a.splits * 4 + mh) * (2 + kDim);
      for (int sp0 = par; sp0 < a.splits; sp0 += 32) {
        float ms[16], ls[16], p0[16], p1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          ms[u] = -INFINITY;
          ls[u] = p0[u] = p1[u] = 0.f;
          if (sp0 + 2 * u < a.splits) {           // uniform: only the splits that exist are read
            const float* s = src + (int64_t)(sp0 + 2 * u) * stride;
            const float2 ml = load_agent2(s), pp = load_agent2(s + 2 + 2 * lane);
            ms[u] = ml.x;
            ls[u] = ml.y;
            p0[u] = pp.x;
            p1[u] = pp.y;
          }
        }
        float mc = M;
#pragma unroll
        for (int u = 0; u < 16; ++u) mc = fmaxf(mc, ms[u]);
        if (mc == -INFINITY) continue;
        const float r = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mc);
        L *= r;
        o0 *= r;
        o1 *= r;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float f = ms[u] != -INFINITY ? __builtin_amdgcn_exp2f(ms[u] - mc) : 0.f;
          L = fmaf(f, ls[u], L);
          o0 = fmaf(f, p0[u], o0);
          o1 = fmaf(f, p1[u], o1);
        }
        M = mc;
      }
    }
    // the odd splits' sums (waves 4..7) join the even ones' (waves 0..3)
    __syncthreads();                           // the wave-merge reads of part_ml / part_o are done
    if (par == 1 && mh < G) {
      if (lane == 0) {
        part_ml[0][mh][0] = M;
        part_ml[0][mh][1] = L;
      }
      part_o[0][mh][2 * lane] = o0;
      part_o[0][mh][2 * lane + 1] = o1;
    }
    __syncthreads();
    if (par == 0 && mh < G) {
      const float m1 = part_ml[0][mh][0];
      const float mc = fmaxf(M, m1);
      if (mc != -INFINITY) {
        const float f0 = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mc);
        const float f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mc);
        L = fmaf(f1, part_ml[0][mh][1], L * f0);
        o0 = fmaf(f1, part_o[0][mh][2 * lane], o0 * f0);
        o1 = fmaf(f1, part_o[0][mh][2 * lane + 1], o1 * f0);
        M = mc;
      }
    }
  }
  float r0 = L > 0.f ? o0 / L : 0.f;
  float r1 = L > 0.f ? o1 / L : 0.f;
  if constexpr (VLM) {
    // Lloyd-Max values were accumulated in the rotated basis: o = diag(s) H o' / sqrt(d).
    float* buf = &part_o[0][0][0] + h * kDim;
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
    float2* o = reinterpret_cast<float2*>(a.out + ((int64_t)b * a.hq + qh0 + h) * kDim);
    o[lane] = make_float2(r0, r1);
  }
}

namespace {

template <int KB, int KM, int VB>
hipError_t decode_v(const DecodeArgs& a, int val_mode, hipStream_t s) {
  const dim3 grid((unsigned)a.splits, (unsigned)(a.hkv * a.hsub), (unsigned)a.batch);
  if (val_mode == TQ_VAL_LLOYD) {
    if constexpr (KB == 8 || KM == kKmPolar) return hipErrorInvalidValue;   // these pair with uniform values
    else hipLaunchKernelGGL((decode_kernel<KB, KM, VB, true>), grid, dim3(64 * kDecodeWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<KB, KM, VB, false>), grid, dim3(64 * kDecodeWaves), 0, s, a);
  }
  return hipGetLastError();
}

template <int KB, int KM>
hipError_t decode_vb(const DecodeArgs& a, int val_bits, int val_mode, hipStream_t s) {
  switch (val_bits) {
    case 2: return decode_v<KB, KM, 2>(a, val_mode, s);
    case 3: return decode_v<KB, KM, 3>(a, val_mode, s);
    case 4: return decode_v<KB, KM, 4>(a, val_mode, s);
  }
  return hipErrorInvalidValue;
}

template <int KB, int KM>
const void* kernel_vb(int val_bits, int val_mode) {
  const bool lm = val_mode == TQ_VAL_LLOYD;
  if constexpr (KB == 8 || KM == kKmPolar) {
    if (lm) return nullptr;
    switch (val_bits) {
      case 2: return (const void*)decode_kernel<KB, KM, 2, false>;
      case 3: return (const void*)decode_kernel<KB, KM, 3, false>;
      case 4: return (const void*)decode_kernel<KB, KM, 4, false>;
    }
    return nullptr;
  } else {
    switch (val_bits) {
      case 2: return lm ? (const void*)decode_kernel<KB, KM, 2, true> : (const void*)decode_kernel<KB, KM, 2, false>;
      case 3: return lm ? (const void*)decode_kernel<KB, KM, 3, true> : (const void*)decode_kernel<KB, KM, 3, false>;
      case 4: return lm ? (const void*)decode_kernel<KB, KM, 4, true> : (const void*)decode_kernel<KB, KM, 4, false>;
    }
    return nullptr;
  }
}

}  // namespace

const void* decode_kernel_ptr(int key_bits, int key_mode, int val_bits, int val_mode) {
  const bool qjl = key_mode == TQ_KEY_LLOYD_QJL;
  if (key_mode == TQ_KEY_POLAR) {
    switch (key_bits) {
      case 2: return kernel_vb<2, kKmPolar>(val_bits, val_mode);
      case 3: return kernel_vb<3, kKmPolar>(val_bits, val_mode);
      case 4: return kernel_vb<4, kKmPolar>(val_bits, val_mode);
    }
    return nullptr;
  }
  switch (key_bits) {
    case 8:
      if (qjl) return nullptr;
      return key_mode == TQ_KEY_FP8 ? kernel_vb<8, kKmFp8>(val_bits, val_mode) : kernel_vb<8, kKmLloyd>(val_bits, val_mode);
    case 2: return qjl ? kernel_vb<2, kKmQjl>(val_bits, val_mode) : kernel_vb<2, kKmLloyd>(val_bits, val_mode);
    case 3: return qjl ? kernel_vb<3, kKmQjl>(val_bits, val_mode) : kernel_vb<3, kKmLloyd>(val_bits, val_mode);
    case 4: return qjl ? kernel_vb<4, kKmQjl>(val_bits, val_mode) : kernel_vb<4, kKmLloyd>(val_bits, val_mode);
  }
  return nullptr;
}

// Scratch of the decode entry point that allocates nothing: the arrival counters
// (kCounterBytes) followed by the split partials, held in device memory for the
// life of the process, one copy per GPU.  Host code reaches it only through the
// device address that scratch_address() returns; the array's name is not a
// device address on the host.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t scratch_address(void** out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

// Zero n 32-bit words (a kernel rather than a memset, so the call stays safe
// to record in a HIP graph).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t s) {
  const int grid = std::max(1, std::min((n + 255) / 256, 64));
  hipLaunchKernelGGL(clear_words_kernel, dim3(grid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int key_bits, int key_mode, int val_bits, int val_mode,
                         hipStream_t s) {
  const bool qjl = key_mode == TQ_KEY_LLOYD_QJL;
  if (key_mode == TQ_KEY_FP8 && key_bits != 8) return hipErrorInvalidValue;
  if (key_mode == TQ_KEY_POLAR) {
    switch (key_bits) {
      case 2: return decode_vb<2, kKmPolar>(a, val_bits, val_mode, s);
      case 3: return decode_vb<3, kKmPolar>(a, val_bits, val_mode, s);
      case 4: return decode_vb<4, kKmPolar>(a, val_bits, val_mode, s);
    }
    return hipErrorInvalidValue;
  }
  switch (key_bits) {
    case 8:
      if (qjl) return hipErrorInvalidValue;
      return key_mode == TQ_KEY_FP8 ? decode_vb<8, kKmFp8>(a, val_bits, val_mode, s)
                                    : decode_vb<8, kKmLloyd>(a, val_bits, val_mode, s);
    case 2: return qjl ? decode_vb<2, kKmQjl>(a, val_bits, val_mode, s) : decode_vb<2, kKmLloyd>(a, val_bits, val_mode, s);
    case 3: return qjl ? decode_vb<3, kKmQjl>(a, val_bits, val_mode, s) : decode_vb<3, kKmLloyd>(a, val_bits, val_mode, s);
    case 4: return qjl ? decode_vb<4, kKmQjl>(a, val_bits, val_mode, s) : decode_vb<4, kKmLloyd>(a, val_bits, val_mode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
