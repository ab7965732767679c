// Host runtime of the C ABI: argument checking, the fp32 Lloyd-Max codebook,
// the page layout, context set-up and launch planning.  All device work is in
// tq_kernels.hip.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "tq_internal.h"

struct tq_ctx {
  tq_config cfg;
  tq_layout layout;
  int device;
  uint32_t sign_bits[4];
  tq::DevConsts* consts;   // device
  float klut_scale, klut_bias, vlut_scale, vlut_bias;
  int unit_grid_ok;        // the page-append key grid resolves every threshold
  int page_wgs;            // page-append grid: resident work-groups on the whole device
  int page_per_cu;         // resident page-append work-groups per compute unit
  int decode_wgs;          // decode grid target: resident work-groups on the whole device
  // Generic path (head_dim 64 / 256): its own
  // constants, S^T for QJL keys, and the device's compute-unit count.
  int generic;
  tq::GenConsts* gconsts;  // device
  float* gSt;              // device [d * d], QJL only
  int cus;
};

namespace {

thread_local std::string g_err;

tq_status fail(tq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

tq_status hip_fail(hipError_t e, const char* what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(uint32_t x) { return x && !(x & (x - 1)); }

// Device address of the static decode scratch, per device (tq_decode_attention_noalloc).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Look up the scratch address of `dev` (the current device) once; nullptr on failure.
void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (tq::scratch_address(&p) == hipSuccess) g_scratch[dev] = p;
    else (void)hipGetLastError();
  }
  return g_scratch[dev];
}

// ---------------------------------------------------------------------------
// Lloyd-Max for a Gaussian coordinate (issoh.co.jp page, stage-1 section:
// per-coordinate Lloyd-Max, representatives placed for the value distribution).
// A rotated unit vector's coordinate is modelled as N(0, 1/d).  Solved for the
// standard normal in long double by alternating the two optimality conditions
// (midpoint thresholds, conditional-mean centroids) from a uniform start.
// ---------------------------------------------------------------------------
long double npdf(long double x) { return std::exp(-0.5L * x * x) * 0.39894228040143267793994605993438L; }
long double ntail(long double x) {  // P(Z > x)
  if (std::isinf(x)) return x > 0 ? 0.0L : 1.0L;
  return 0.5L * std::erfc(x * 0.70710678118654752440084436210485L);
}

void lloyd_max_std(int bits, std::vector<double>& centroids, std::vector<double>& thresholds) {
  const int levels = 1 << bits, half = levels / 2;
  std::vector<long double> c(half);       // positive centroids, ascending
  for (int i = 0; i < half; ++i) c[i] = (i + 0.5L) * 3.0L / half;
  std::vector<long double> t(half + 1);
  // With many levels the alternation contracts its error only by about
  // 1 - O(1/k^2) per round: from 5 bits on, a bounded number of rounds is followed
  // by Newton's method on the same equations (below).
  const int rounds = bits <= 4 ? 200000 : 2000;
  for (int it = 0; it < rounds; ++it) {
    t[0] = 0.0L;
    t[half] = std::numeric_limits<long double>::infinity();
    for (int i = 1; i < half; ++i) t[i] = 0.5L * (c[i - 1] + c[i]);
    long double moved = 0.0L;
    for (int i = 0; i < half; ++i) {
      long double mass = ntail(t[i]) - ntail(t[i + 1]);
      long double num = npdf(t[i]) - (std::isinf(t[i + 1]) ? 0.0L : npdf(t[i + 1]));
      long double nc = num / mass;
      moved = std::fmax(moved, std::fabs(nc - c[i]));
      c[i] = nc;
    }
    if (moved < 1e-17L) break;
  }
  if (bits > 4) {
    // Newton on G(c) = c - m(c): the mean of a cell moves with its edges as
    // dm/da = phi(a)(m - a)/P and dm/db = phi(b)(b - m)/P, and the edges are the
    // midpoints of neighbouring centroids, so the Jacobian is tridiagonal
    // (solved by elimination down the diagonal).
    std::vector<long double> lo(half), di(half), up(half), g(half);
    for (int step = 0; step < 60; ++step) {
      long double worst = 0.0L;
      for (int i = 0; i < half; ++i) {
        const long double a = i == 0 ? 0.0L : 0.5L * (c[i - 1] + c[i]);
        const bool last = i == half - 1;
        const long double b = last ? std::numeric_limits<long double>::infinity() : 0.5L * (c[i] + c[i + 1]);
        const long double P = ntail(a) - ntail(b);
        const long double m = (npdf(a) - (last ? 0.0L : npdf(b))) / P;
        const long double dA = i == 0 ? 0.0L : npdf(a) * (m - a) / P;
        const long double dB = last ? 0.0L : npdf(b) * (b - m) / P;
        g[i] = c[i] - m;
        di[i] = 1.0L - 0.5L * dA - 0.5L * dB;
        lo[i] = -0.5L * dA;
        up[i] = -0.5L * dB;
      }
      for (int i = 1; i < half; ++i) {   // forward elimination
        const long double f = lo[i] / di[i - 1];
        di[i] -= f * up[i - 1];
        g[i] -= f * g[i - 1];
      }
      for (int i = half - 1; i >= 0; --i) {   // back substitution: g becomes the step
        g[i] = (g[i] - (i + 1 < half ? up[i] * g[i + 1] : 0.0L)) / di[i];
        c[i] -= g[i];
        worst = std::fmax(worst, std::fabs(g[i]));
      }
      if (worst < 1e-17L) break;
    }
  }
  centroids.assign(levels, 0.0);
  thresholds.assign(levels - 1, 0.0);
  for (int i = 0; i < half; ++i) {
    centroids[half + i] = (double)c[i];
    centroids[half - 1 - i] = -(double)c[i];
  }
  for (int i = 1; i < half; ++i) {
    double m = (double)(0.5L * (c[i - 1] + c[i]));
    thresholds[half - 1 + i] = m;
    thresholds[half - 1 - i] = -m;
  }
  thresholds[half - 1] = 0.0;
}

void codebook_f32(int bits, int d, float* c, float* t) {
  std::vector<double> cd, td;
  lloyd_max_std(bits, cd, td);
  const double s = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < (1 << bits); ++i) c[i] = (float)(cd[i] * s);
  for (int i = 0; i < (1 << bits) - 1; ++i) t[i] = (float)(td[i] * s);
}

// Uniform grid over [-range, range) that resolves every fp32 threshold with one
// comparison.  range is a power of two so that y * scale is exact.
bool build_lut(int bits, const float* c, const float* t, tq::QLut* lut, float* scale, float* bias) {
  const int nt = (1 << bits) - 1;
  double tmax = 0;
  for (int i = 0; i < nt; ++i) tmax = std::fmax(tmax, std::fabs((double)t[i]));
  double range = 1.0 / 64;
  while (range < 1.1 * tmax) range *= 2;
  const int cells = tq::kLutCells;
  const double w = 2 * range / cells;
  for (int k = 0; k < cells; ++k) {
    double lo = (k == 0) ? -INFINITY : -range + k * w - 0.25 * w;
    double hi = (k == cells - 1) ? INFINITY : -range + (k + 1) * w + 0.25 * w;
    int base = 0, inside = 0;
    float tin = INFINITY;
    for (int j = 0; j < nt; ++j) {
      if ((double)t[j] < lo) ++base;
      else if ((double)t[j] <= hi) { ++inside; tin = t[j]; }
    }
    if (inside > 1) return false;
    lut[k].base = base;
    lut[k].t = tin;
    lut[k].c_lo = c[base];
    lut[k].c_hi = c[base + 1 <= nt ? base + 1 : nt];
  }
  *scale = (float)((cells / 2) / range);
  *bias = (float)(cells / 2);
  return true;
}

// Grid of the page kernel over g = 128 y, |y| <= 1: cell k (0..256) takes g in
// [k - 128.5, k - 127.5) widened by a quarter cell on each side (the end cells
// reach to infinity), so that a cell found from a slightly rounded g still holds
// the right answer; at most one threshold may fall inside a widened cell.
// Thresholds are stored as 128 t (exact: a power-of-two scaling).
bool build_unit_lut(int bits, const float* c, const float* t, tq::QLut* lut) {
  const int nt = (1 << bits) - 1;
  for (int k = 0; k < tq::kUnitCellsPadded; ++k) {
    const int kk = std::min(k, tq::kUnitCells - 1);
    const double lo = (kk == 0) ? -INFINITY : kk - 128.75;
    const double hi = (kk == tq::kUnitCells - 1) ? INFINITY : kk - 127.25;
    int base = 0, inside = 0;
    float tin = INFINITY;
    for (int j = 0; j < nt; ++j) {
      const double tg = 128.0 * (double)t[j];
      if (tg < lo) ++base;
      else if (tg <= hi) { ++inside; tin = 128.0f * t[j]; }
    }
    if (inside > 1) return false;
    lut[k].base = base;
    lut[k].t = tin;
    lut[k].c_lo = c[base];
    lut[k].c_hi = c[base + 1 <= nt ? base + 1 : nt];
  }
  return true;
}

// The tuned kernels take head_dim 128 with any group size (up to the group limit);
// the decode takes the query heads of a KV head in head groups of up to 4.
bool is_generic(const tq_config* c) { return c->head_dim != (uint32_t)tq::kDim; }

// Query heads per KV head and head groups per KV head of the tuned decode.
void tuned_groups(const tq_config& c, int* group, int* hsub) {
  const int g = (int)(c.num_q_heads / c.num_kv_heads);
  *group = g;
  *hsub = (g + 3) / 4;
}

tq_status layout_of(const tq_config* c, tq_layout* L) {
  const size_t T = TQ_BLOCK_TOKENS, d = c->head_dim;
  std::memset(L, 0, sizeof *L);
  L->format_version = TQ_FORMAT_VERSION;
  const size_t none = (size_t)-1;
  size_t off = 0;
  L->off_kcodes = off; L->row_kcodes = d * c->key_bits / 8; off += T * L->row_kcodes;
  if (c->key_mode == TQ_KEY_FP8) {
    L->off_knorm = none;
  } else {
    L->off_knorm = off; off += T * 4;
  }
  if (c->key_mode == TQ_KEY_LLOYD_QJL) {
    L->off_ksigns = off; L->row_ksigns = d / 8; off += T * L->row_ksigns;
    L->off_kresid = off; off += T * 4;
  } else {
    L->off_ksigns = none; L->row_ksigns = 0; L->off_kresid = none;
  }
  L->off_vcodes = off; L->row_vcodes = d * c->val_bits / 8; off += T * L->row_vcodes;
  L->off_vmin = off; off += T * 4;
  if (c->val_mode == TQ_VAL_UNIFORM) { L->off_vscale = off; off += T * 4; } else L->off_vscale = none;
  L->page_bytes = off;
  L->token_head_bytes = off / T;
  const size_t limit = is_generic(c) ? (size_t)tq::kGenMaxPageBytes : (size_t)tq::kMaxPageBytes;
  if (off > limit) return fail(TQ_ERR_UNSUPPORTED, "page of %zu bytes exceeds %zu", off, limit);
  return TQ_OK;
}

tq::FieldOffsets offsets_of(const tq_layout& L) {
  tq::FieldOffsets f;
  f.page_bytes = (uint32_t)L.page_bytes;
  f.kcodes = (uint32_t)L.off_kcodes;
  f.knorm = L.off_knorm == (size_t)-1 ? 0u : (uint32_t)L.off_knorm;
  f.ksigns = L.off_ksigns == (size_t)-1 ? 0u : (uint32_t)L.off_ksigns;
  f.kres = L.off_kresid == (size_t)-1 ? 0u : (uint32_t)L.off_kresid;
  f.vcodes = (uint32_t)L.off_vcodes;
  f.vmin = (uint32_t)L.off_vmin;
  f.vscale = L.off_vscale == (size_t)-1 ? 0u : (uint32_t)L.off_vscale;
  return f;
}

// Split the context of every (sequence, kv head) into `splits` even shares of
// whole 64-token tiles so that the grid is about one round of resident
// work-groups (`target`, from the kernel's occupancy): more, shorter splits only
// add prologues and merges, fewer leave SIMDs idle.  A split holds 4 to 64 tiles.
// Generic decode: splits of whole 64-token blocks, about `target` work-groups in
// all, at most 64 splits per (sequence, KV head).
// Splits of the generic decode: whole 64-token blocks per split, one 4-wave
// work-group each.  Each wave should get about two blocks (four at head_dim 64,
// whose blocks are cheap next to a work-group's prologue: the query rotation and
// the tables), with at most 4 * target work-groups in the grid and 64 splits.
void plan_gen_splits(int target, int batch, int hkv, int max_seq, int head_dim, int* splits, int* chunk,
                     int max_splits = 64) {
  constexpr int kWaves = 4;
  const int blocks = std::max(1, (max_seq + 63) / 64);
  const int64_t pairs = std::max<int64_t>(1, (int64_t)batch * hkv);
  const int per_wave = head_dim == 64 ? 4 : 2;
  const int64_t by_grid = std::max<int64_t>(1, (4 * (int64_t)target + pairs - 1) / pairs);
  const int64_t by_work = std::max(1, (blocks + per_wave * kWaves - 1) / (per_wave * kWaves));
  int want = (int)std::min<int64_t>(std::min<int64_t>(blocks, by_grid),
                                    std::min<int64_t>(by_work, std::max(1, std::min(max_splits, 64))));
  const int per = (blocks + want - 1) / want;
  *chunk = per * 64;
  *splits = (blocks + per - 1) / per;
}

void plan_splits(int target, int batch, int hkv, int max_seq, int* splits, int* tiles_total) {
  const int tiles = std::max(1, (max_seq + 63) / 64);
  const int pairs = std::max(1, batch * hkv);
  int want = (target + pairs - 1) / pairs;
  want = std::max(1, std::min(want, (tiles + 3) / 4));
  want = std::max(want, (tiles + tq::kMaxPagesPerSplit / 4 - 1) / (tq::kMaxPagesPerSplit / 4));
  *splits = want;
  *tiles_total = tiles;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) hipSetDevice(prev);
  }
};

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Context of a generic-path configuration (validated by the caller): the
// codebooks, signs and S^T on the device.
tq_status create_generic(const tq_config* cfg, const int8_t* signs_host, const float* S_host, tq_ctx** out) {
  const int d = (int)cfg->head_dim;
  tq::GenConsts h;
  std::memset(&h, 0, sizeof h);
  for (int i = 0; i < d; ++i) h.signs[i] = (float)signs_host[i];
  if (cfg->key_mode == TQ_KEY_FP8) {
    // the value of every E4M3 byte (sign, 4 exponent bits with bias 7, 3 mantissa bits;
    // exponent 0 holds m * 2^-9; S.1111.111 is NaN and never written)
    for (int code = 0; code < 256; ++code) {
      const int e = (code >> 3) & 15, m = code & 7;
      const double mag = e == 0 ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
      h.kc[code] = (code & 0x7F) == 0x7F ? std::numeric_limits<float>::quiet_NaN() : (float)((code & 0x80) ? -mag : mag);
    }
  } else {
    codebook_f32((int)cfg->key_bits, d, h.kc, h.kt);
  }
  if (cfg->val_mode == TQ_VAL_LLOYD) codebook_f32((int)cfg->val_bits, d, h.vc, h.vt);
  std::vector<float> st;
  if (cfg->key_mode == TQ_KEY_LLOYD_QJL) {
    st.resize((size_t)d * d);
    for (int m = 0; m < d; ++m)
      for (int k = 0; k < d; ++k) st[(size_t)k * d + m] = S_host[(size_t)m * d + k];
  }
  tq_ctx* ctx = new (std::nothrow) tq_ctx();
  if (!ctx) return fail(TQ_ERR_OUT_OF_MEMORY, "host allocation failed");
  ctx->cfg = *cfg;
  tq_status s = layout_of(cfg, &ctx->layout);
  if (s != TQ_OK) { delete ctx; return s; }
  ctx->generic = 1;
  ctx->consts = nullptr;
  ctx->gconsts = nullptr;
  ctx->gSt = nullptr;
  for (int i = 0; i < 4; ++i) ctx->sign_bits[i] = 0;
  hipError_t e = hipGetDevice(&ctx->device);
  if (e != hipSuccess) { delete ctx; return hip_fail(e, "hipGetDevice"); }
  e = hipMalloc((void**)&ctx->gconsts, sizeof(tq::GenConsts));
  if (e == hipSuccess) e = hipMemcpy(ctx->gconsts, &h, sizeof h, hipMemcpyHostToDevice);
  if (e == hipSuccess && !st.empty()) {
    e = hipMalloc((void**)&ctx->gSt, st.size() * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(ctx->gSt, st.data(), st.size() * sizeof(float), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    if (ctx->gconsts) hipFree(ctx->gconsts);
    if (ctx->gSt) hipFree(ctx->gSt);
    delete ctx;
    return e == hipErrorOutOfMemory ? fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc") : hip_fail(e, "generic constants upload");
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, ctx->device) != hipSuccess || cus <= 0)
    cus = 256;
  (void)hipGetLastError();
  ctx->cus = cus;
  ctx->decode_wgs = 2 * cus;
  ctx->page_wgs = 8 * cus;
  ctx->page_per_cu = 0;
  ctx->klut_scale = ctx->klut_bias = ctx->vlut_scale = ctx->vlut_bias = 0.f;
  ctx->unit_grid_ok = 0;
  (void)scratch_of(ctx->device);   // the no-allocation decode's scratch on this device
  *out = ctx;
  return TQ_OK;
}

tq::GenRows gen_rows(const tq_layout& L) {
  tq::GenRows r;
  r.kcodes = (uint32_t)L.row_kcodes;
  r.ksigns = (uint32_t)L.row_ksigns;
  r.vcodes = (uint32_t)L.row_vcodes;
  return r;
}

// generic kernels' key mode: 0 plain Lloyd-Max, 1 corrected norm, 2 QJL, 3 FP8
int gen_key_mode(const tq_config& c) {
  return c.key_mode == TQ_KEY_LLOYD_NC ? 1 : c.key_mode == TQ_KEY_LLOYD_QJL ? 2 : c.key_mode == TQ_KEY_FP8 ? 3 : 0;
}

}  // namespace

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_WORKSPACE_TOO_SMALL: return "TQ_ERR_WORKSPACE_TOO_SMALL";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_OUT_OF_MEMORY: return "TQ_ERR_OUT_OF_MEMORY";
  }
  return "TQ_ERR_UNKNOWN";
}

const char* tq_last_error_message(void) { return g_err.c_str(); }

tq_status tq_validate_config(const tq_config* c) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "cfg is null");
  if (c->abi_version != TQ_ABI_VERSION) return fail(TQ_ERR_INVALID_ARG, "abi_version %u != %d", c->abi_version, TQ_ABI_VERSION);
  if (c->block_tokens != TQ_BLOCK_TOKENS) return fail(TQ_ERR_INVALID_ARG, "block_tokens must be %d", TQ_BLOCK_TOKENS);
  if (!is_pow2(c->head_dim) || c->head_dim < 8 || c->head_dim > 1024)
    return fail(TQ_ERR_INVALID_ARG, "head_dim %u is not a power of two in [8, 1024]", c->head_dim);
  if (c->num_kv_heads == 0 || c->num_q_heads == 0 || c->num_q_heads % c->num_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "num_q_heads (%u) must be a positive multiple of num_kv_heads (%u)",
                c->num_q_heads, c->num_kv_heads);
  if (c->key_mode > TQ_KEY_POLAR) return fail(TQ_ERR_INVALID_ARG, "bad key_mode %u", c->key_mode);
  if (c->val_mode > TQ_VAL_LLOYD) return fail(TQ_ERR_INVALID_ARG, "bad val_mode %u", c->val_mode);
  if (c->key_bits < 1 || c->key_bits > 8) return fail(TQ_ERR_INVALID_ARG, "key_bits %u out of [1, 8]", c->key_bits);
  if (c->val_bits < 1 || c->val_bits > 8) return fail(TQ_ERR_INVALID_ARG, "val_bits %u out of [1, 8]", c->val_bits);
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %u: supported 64, 128 (tuned) and 256", c->head_dim);
  const uint32_t g = c->num_q_heads / c->num_kv_heads;
  if (g > (uint32_t)tq::kGenMaxGroup)
    return fail(TQ_ERR_UNSUPPORTED, "group size %u: supported 1..%d", g, tq::kGenMaxGroup);
  if (is_generic(c) && c->key_mode == TQ_KEY_POLAR)
    return fail(TQ_ERR_UNSUPPORTED, "PolarQuant keys are built for head_dim 128");
  if (c->key_mode == TQ_KEY_FP8) {
    if (c->key_bits != 8) return fail(TQ_ERR_INVALID_ARG, "FP8 keys take key_bits 8 (got %u)", c->key_bits);
    if (c->val_mode != TQ_VAL_UNIFORM) return fail(TQ_ERR_UNSUPPORTED, "FP8 keys are built with uniform values only");
  } else if (c->key_mode == TQ_KEY_POLAR) {
    if (c->key_bits < 2 || c->key_bits > 4) return fail(TQ_ERR_UNSUPPORTED, "PolarQuant keys take 2..4 bits per angle");
    if (c->val_mode != TQ_VAL_UNIFORM) return fail(TQ_ERR_UNSUPPORTED, "PolarQuant keys are built with uniform values only");
  } else if (c->key_bits == 8) {
    if (c->key_mode == TQ_KEY_LLOYD_QJL) return fail(TQ_ERR_UNSUPPORTED, "8-bit keys take no QJL residual");
  } else if (c->key_bits < 2 || c->key_bits > 4) {
    return fail(TQ_ERR_UNSUPPORTED, "key_bits %u: supported 2..4 and 8", c->key_bits);
  }
  if (c->val_bits < 2 || c->val_bits > 4) return fail(TQ_ERR_UNSUPPORTED, "val_bits %u: supported 2..4", c->val_bits);
  if (c->num_kv_heads > 65535) return fail(TQ_ERR_UNSUPPORTED, "num_kv_heads too large");
  return TQ_OK;
}

tq_status tq_layout_for_config(const tq_config* cfg, tq_layout* out) {
  tq_status s = tq_validate_config(cfg);
  if (s != TQ_OK) return s;
  if (!out) return fail(TQ_ERR_INVALID_ARG, "out is null");
  return layout_of(cfg, out);
}

tq_status tq_codebook(uint32_t bits, uint32_t head_dim, float* centroids, float* thresholds) {
  if (bits < 1 || bits > 8 || !is_pow2(head_dim) || !centroids || !thresholds)
    return fail(TQ_ERR_INVALID_ARG, "bad codebook request (bits %u, head_dim %u)", bits, head_dim);
  codebook_f32((int)bits, (int)head_dim, centroids, thresholds);
  return TQ_OK;
}

tq_status tq_create(const tq_config* cfg, const int8_t* signs_host, const float* S_host, tq_ctx** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  tq_status s = tq_validate_config(cfg);
  if (s != TQ_OK) return s;
  if (!signs_host) return fail(TQ_ERR_INVALID_ARG, "signs_host is null");
  const int d = (int)cfg->head_dim;
  for (int i = 0; i < d; ++i)
    if (signs_host[i] != 1 && signs_host[i] != -1) return fail(TQ_ERR_INVALID_ARG, "signs_host[%d] = %d is not +-1", i, signs_host[i]);
  if (cfg->key_mode == TQ_KEY_LLOYD_QJL && !S_host) return fail(TQ_ERR_INVALID_ARG, "QJL keys need qjl_S_host");
  if (is_generic(cfg)) return create_generic(cfg, signs_host, S_host, out);

  tq::DevConsts* h = new (std::nothrow) tq::DevConsts();
  if (!h) return fail(TQ_ERR_OUT_OF_MEMORY, "host allocation failed");
  std::memset(h, 0, sizeof *h);
  for (int i = 0; i < d; ++i) h->signs[i] = (float)signs_host[i];
  float vt[15] = {0};
  const bool fp8 = cfg->key_mode == TQ_KEY_FP8;   // no key codebook
  const bool polar = cfg->key_mode == TQ_KEY_POLAR;
  const bool wide = cfg->key_bits > 4;            // 8-bit codes: a binary search over h->kt, no grid
  if (!fp8 && !polar) codebook_f32((int)cfg->key_bits, d, h->kc, h->kt);
  if (polar) {
    // cell centres of the angle grids: level 1 over [-pi, pi), levels >= 2 over [0, pi/2]
    const double pi = std::acos(-1.0);
    const int n = 1 << cfg->key_bits;
    for (int c = 0; c < n; ++c) {
      const double t1 = -pi + (c + 0.5) * (2 * pi / n), tu = (c + 0.5) * (0.5 * pi / n);
      h->pcs1[2 * c] = (float)std::cos(t1); h->pcs1[2 * c + 1] = (float)std::sin(t1);
      h->pcsU[2 * c] = (float)std::cos(tu); h->pcsU[2 * c + 1] = (float)std::sin(tu);
    }
  }
  const float* kt = h->kt;
  tq_ctx* ctx = new (std::nothrow) tq_ctx();
  if (!ctx) { delete h; return fail(TQ_ERR_OUT_OF_MEMORY, "host allocation failed"); }
  ctx->cfg = *cfg;
  if ((s = layout_of(cfg, &ctx->layout)) != TQ_OK) { delete h; delete ctx; return s; }
  bool ok = fp8 || polar || wide || build_lut((int)cfg->key_bits, h->kc, kt, h->klut, &ctx->klut_scale, &ctx->klut_bias);
  ctx->unit_grid_ok = (!fp8 && !polar && !wide && build_unit_lut((int)cfg->key_bits, h->kc, kt, h->kulut)) ? 1 : 0;
  if (cfg->val_mode == TQ_VAL_LLOYD) {
    codebook_f32((int)cfg->val_bits, d, h->vc, vt);
    ok = ok && build_lut((int)cfg->val_bits, h->vc, vt, h->vlut, &ctx->vlut_scale, &ctx->vlut_bias);
  }
  if (!ok) { delete h; delete ctx; return fail(TQ_ERR_UNSUPPORTED, "codebook thresholds too dense for the look-up grid"); }
  if (cfg->key_mode == TQ_KEY_LLOYD_QJL) {
    for (int m = 0; m < d; ++m)
      for (int k = 0; k < d; ++k) h->St[k * d + m] = S_host[m * d + k];
    for (int mt = 0; mt < 8; ++mt)
      for (int n = 0; n < 4; ++n)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const float x = S_host[(16 * mt + l % 16) * d + 32 * n + 8 * (l / 16) + e];
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            const uint32_t sh = 16u * (uint32_t)(e & 1);
            const size_t w = ((size_t)((0 * 8 + mt) * 4 + n) * 64 + l) * 4 + e / 2;
            const size_t w_lo = ((size_t)((1 * 8 + mt) * 4 + n) * 64 + l) * 4 + e / 2;
            h->Sh[w] |= (uint32_t)__builtin_bit_cast(uint16_t, hi) << sh;
            h->Sh[w_lo] |= (uint32_t)__builtin_bit_cast(uint16_t, lo) << sh;
          }
  }
  for (int i = 0; i < 4; ++i) ctx->sign_bits[i] = 0;
  for (int i = 0; i < d; ++i)
    if (signs_host[i] < 0) ctx->sign_bits[i >> 5] |= 1u << (i & 31);

  hipError_t e = hipGetDevice(&ctx->device);
  if (e != hipSuccess) { delete h; delete ctx; return hip_fail(e, "hipGetDevice"); }
  e = hipMalloc((void**)&ctx->consts, sizeof(tq::DevConsts));
  if (e != hipSuccess) { delete h; delete ctx; return e == hipErrorOutOfMemory ? fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc") : hip_fail(e, "hipMalloc"); }
  e = hipMemcpy(ctx->consts, h, sizeof(tq::DevConsts), hipMemcpyHostToDevice);
  delete h;
  if (e != hipSuccess) { hipFree(ctx->consts); delete ctx; return hip_fail(e, "hipMemcpy"); }
  // Decode grid target: kDecodeWgsPerCu work-groups per compute unit (fewer if
  // fewer fit), all resident at once.
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, tq::decode_kernel_ptr((int)cfg->key_bits, (int)cfg->key_mode, (int)cfg->val_bits,
                                         (int)cfg->val_mode),
          64 * tq::kDecodeWaves, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  per_cu = std::min(per_cu, tq::kDecodeWgsPerCu);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, ctx->device) != hipSuccess || cus <= 0)
    cus = 256;
  (void)hipGetLastError();
  ctx->decode_wgs = per_cu * cus;
  int page_per_cu = 0;
  const void* pk = tq::append_page_kernel_ptr((int)cfg->key_bits, (int)cfg->val_bits,
                                              cfg->key_mode == TQ_KEY_LLOYD_QJL);
  if (!pk || hipOccupancyMaxActiveBlocksPerMultiprocessor(&page_per_cu, pk, 256, 0) != hipSuccess || page_per_cu <= 0)
    page_per_cu = 2;
  (void)hipGetLastError();
  ctx->page_wgs = page_per_cu * cus;
  ctx->page_per_cu = page_per_cu;
  ctx->generic = 0;
  ctx->gconsts = nullptr;
  ctx->gSt = nullptr;
  ctx->cus = cus;
  (void)scratch_of(ctx->device);   // set-up of the no-allocation decode's scratch on this device
  *out = ctx;
  return TQ_OK;
}

void tq_destroy(tq_ctx* ctx) {
  if (!ctx) return;
  DeviceGuard g(ctx->device);
  if (ctx->consts) hipFree(ctx->consts);
  if (ctx->gconsts) hipFree(ctx->gconsts);
  if (ctx->gSt) hipFree(ctx->gSt);
  delete ctx;
}

tq_status tq_layout_query(const tq_ctx* ctx, tq_layout* out) {
  if (!ctx || !out) return fail(TQ_ERR_INVALID_ARG, "null argument");
  *out = ctx->layout;
  return TQ_OK;
}

tq_status tq_quantize_append(tq_ctx* ctx, const void* k, const void* v, tq_dtype dt, int64_t num_tokens,
                             const int64_t* slot_mapping, void* cache, int64_t num_blocks, hipStream_t stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "ctx is null");
  if (dt != TQ_F32 && dt != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  if (num_tokens < 0 || num_blocks < 0) return fail(TQ_ERR_INVALID_ARG, "negative size");
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !cache) return fail(TQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(cache, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
    return fail(TQ_ERR_INVALID_ARG, "k, v and cache must be 16-byte aligned");
  if (num_tokens * (int64_t)ctx->cfg.num_kv_heads > ((int64_t)1 << 38))
    return fail(TQ_ERR_UNSUPPORTED, "num_tokens * num_kv_heads too large for one launch");
  DeviceGuard g(ctx->device);
  if (ctx->generic) {
    tq::GenAppendArgs ga;
    std::memset(&ga, 0, sizeof ga);
    ga.k = k; ga.v = v; ga.bf16 = dt == TQ_BF16; ga.num_tokens = num_tokens; ga.hkv = (int32_t)ctx->cfg.num_kv_heads;
    ga.key_bits = (int32_t)ctx->cfg.key_bits; ga.key_mode = gen_key_mode(ctx->cfg);
    ga.val_bits = (int32_t)ctx->cfg.val_bits; ga.val_mode = ctx->cfg.val_mode == TQ_VAL_LLOYD ? 1 : 0;
    ga.slots = slot_mapping; ga.cache = (uint8_t*)cache; ga.num_blocks = num_blocks;
    ga.f = offsets_of(ctx->layout); ga.rows = gen_rows(ctx->layout); ga.c = ctx->gconsts; ga.St = ctx->gSt;
    hipError_t ge = tq::launch_gen_append(ga, (int)ctx->cfg.head_dim, ctx->page_wgs, stream);
    return ge == hipSuccess ? TQ_OK : hip_fail(ge, "append launch");
  }
  tq::AppendArgs a;
  a.k = k; a.v = v; a.num_tokens = num_tokens; a.hkv = (int32_t)ctx->cfg.num_kv_heads;
  for (int i = 0; i < 4; ++i) a.sign_bits[i] = ctx->sign_bits[i];
  a.key_nc = ctx->cfg.key_mode == TQ_KEY_LLOYD_NC;
  a.slots = slot_mapping; a.cache = (uint8_t*)cache; a.num_blocks = num_blocks;
  a.f = offsets_of(ctx->layout); a.c = ctx->consts;
  a.klut_scale = ctx->klut_scale; a.klut_bias = ctx->klut_bias;
  a.vlut_scale = ctx->vlut_scale; a.vlut_bias = ctx->vlut_bias;
  a.unit_grid_ok = ctx->unit_grid_ok;
  a.page_wgs = ctx->page_wgs;
  a.page_per_cu = ctx->page_per_cu;
  hipError_t e = tq::launch_append(a, (int)dt, (int)ctx->cfg.key_bits, (int)ctx->cfg.key_mode,
                                   (int)ctx->cfg.val_bits, (int)ctx->cfg.val_mode, stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "append launch");
}

size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t max_seq_len) {
  if (!ctx || batch <= 0 || max_seq_len < 0) return 0;
  if (ctx->generic) {
    int splits, chunk;
    plan_gen_splits(ctx->decode_wgs, batch, (int)ctx->cfg.num_kv_heads, max_seq_len, (int)ctx->cfg.head_dim,
                    &splits, &chunk);
    return tq::kCounterBytes + (size_t)batch * ctx->cfg.num_q_heads * splits * (2 + ctx->cfg.head_dim) * sizeof(float);
  }
  int splits, tps, group, hsub;
  tuned_groups(ctx->cfg, &group, &hsub);
  plan_splits(ctx->decode_wgs, batch, (int)ctx->cfg.num_kv_heads * hsub, max_seq_len, &splits, &tps);
  return tq::kCounterBytes +
         (size_t)batch * ctx->cfg.num_kv_heads * hsub * splits * tq::kMaxGroup * (2 + tq::kDim) * sizeof(float);
}

namespace {

tq_status decode_common(tq_ctx* ctx, const void* q, tq_dtype dt, const void* cache, int64_t num_blocks,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                        int32_t batch, int32_t max_seq_len, float softmax_scale, float* out, float* logits_out,
                        void* workspace, size_t workspace_bytes, const void* k_new, const void* v_new,
                        hipStream_t stream, bool static_scratch = false) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "ctx is null");
  if (dt != TQ_F32 && dt != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  if (batch < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(TQ_ERR_INVALID_ARG, "negative size");
  if (!std::isfinite(softmax_scale)) return fail(TQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (batch == 0) return TQ_OK;
  if (batch > 65535) return fail(TQ_ERR_UNSUPPORTED, "batch > 65535");
  int group = 0, hsub = 1;   // tuned decode: query heads per work-group, work-groups per KV head
  if (!ctx->generic) tuned_groups(ctx->cfg, &group, &hsub);
  if ((size_t)batch * ctx->cfg.num_kv_heads * hsub * sizeof(uint32_t) > tq::kCounterBytes)
    return fail(TQ_ERR_UNSUPPORTED, "batch * num_kv_heads * (query heads per KV head / 4) > %zu",
                tq::kCounterBytes / sizeof(uint32_t));
  if (!q || !cache || !block_tables || !seq_lens || !out || (!workspace && !static_scratch))
    return fail(TQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(cache, 16) || (!static_scratch && !aligned(workspace, 16)) || !aligned(q, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (cache/workspace need 16 bytes)");
  if (k_new != nullptr) {
    if (!v_new) return fail(TQ_ERR_INVALID_ARG, "v_new is null");
    if (!aligned(k_new, 4) || !aligned(v_new, 4)) return fail(TQ_ERR_INVALID_ARG, "misaligned k_new / v_new");
    if (ctx->cfg.val_mode == TQ_VAL_LLOYD && !ctx->generic)
      return fail(TQ_ERR_UNSUPPORTED, "the fused append takes uniform values only");
  }
  // The generic decode in the static scratch plans no more splits than its
  // partials can hold there (a different split count changes only the fp32
  // summation order).
  int gen_max_splits = 64;
  size_t need = tq_decode_workspace_bytes(ctx, batch, max_seq_len);
  if (ctx->generic && static_scratch) {
    const size_t per_split = (size_t)batch * ctx->cfg.num_q_heads * (2 + ctx->cfg.head_dim) * sizeof(float);
    const size_t fit = (tq::kStaticScratchBytes - tq::kCounterBytes) / per_split;
    gen_max_splits = (int)std::min<size_t>(fit, 64);
    int splits, chunk;
    plan_gen_splits(ctx->decode_wgs, batch, (int)ctx->cfg.num_kv_heads, max_seq_len, (int)ctx->cfg.head_dim,
                    &splits, &chunk, std::max(1, gen_max_splits));
    need = tq::kCounterBytes + (size_t)splits * per_split;
  }
  if (static_scratch && need > tq::kStaticScratchBytes)
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "batch %d x %u kv heads up to %d tokens needs %zu bytes of scratch; "
                "the static scratch holds %zu", batch, ctx->cfg.num_kv_heads, max_seq_len, need,
                tq::kStaticScratchBytes);
  if (!static_scratch && workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  DeviceGuard g(ctx->device);
  if (static_scratch) {
    workspace = scratch_of(ctx->device);
    if (!workspace) return fail(TQ_ERR_HIP, "no device address for the static scratch on device %d", ctx->device);
    workspace_bytes = tq::kStaticScratchBytes;
  }
  if (ctx->generic) {
    const int hkv = (int)ctx->cfg.num_kv_heads, G = (int)(ctx->cfg.num_q_heads / ctx->cfg.num_kv_heads);
    const int d = (int)ctx->cfg.head_dim;
    if (k_new != nullptr) {
      // the new tokens first (one launch), then the decode over the context including them
      tq::GenAppendArgs ga;
      std::memset(&ga, 0, sizeof ga);
      ga.k = k_new; ga.v = v_new; ga.bf16 = dt == TQ_BF16; ga.num_tokens = batch; ga.hkv = hkv;
      ga.key_bits = (int32_t)ctx->cfg.key_bits; ga.key_mode = gen_key_mode(ctx->cfg);
      ga.val_bits = (int32_t)ctx->cfg.val_bits; ga.val_mode = ctx->cfg.val_mode == TQ_VAL_LLOYD ? 1 : 0;
      ga.slots = nullptr; ga.block_tables = block_tables; ga.max_blocks = max_blocks_per_seq; ga.seq_lens = seq_lens;
      ga.max_seq = max_seq_len; ga.cache = (uint8_t*)const_cast<void*>(cache); ga.num_blocks = num_blocks;
      ga.f = offsets_of(ctx->layout); ga.rows = gen_rows(ctx->layout); ga.c = ctx->gconsts; ga.St = ctx->gSt;
      hipError_t ge = tq::launch_gen_append(ga, d, ctx->page_wgs, stream);
      if (ge != hipSuccess) return hip_fail(ge, "append launch");
    }
    tq::GenDecodeArgs ga;
    std::memset(&ga, 0, sizeof ga);
    ga.q = q; ga.q_bf16 = dt == TQ_BF16; ga.cache = (const uint8_t*)cache; ga.num_blocks = num_blocks;
    ga.block_tables = block_tables; ga.max_blocks = max_blocks_per_seq; ga.seq_lens = seq_lens;
    ga.batch = batch; ga.max_seq = max_seq_len; ga.hkv = hkv; ga.group = G;
    ga.key_bits = (int32_t)ctx->cfg.key_bits; ga.key_mode = gen_key_mode(ctx->cfg);
    ga.val_bits = (int32_t)ctx->cfg.val_bits; ga.val_mode = ctx->cfg.val_mode == TQ_VAL_LLOYD ? 1 : 0;
    ga.scale = softmax_scale; ga.qjl_coef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / d);
    ga.logits = logits_out; ga.out = out;
    ga.ws = (float*)((uint8_t*)workspace + tq::kCounterBytes);
    plan_gen_splits(ctx->decode_wgs, batch, hkv, max_seq_len, d, &ga.splits, &ga.chunk, std::max(1, gen_max_splits));
    ga.f = offsets_of(ctx->layout); ga.rows = gen_rows(ctx->layout); ga.c = ctx->gconsts; ga.St = ctx->gSt;
    hipError_t ge = tq::launch_gen_decode(ga, d, stream);
    return ge == hipSuccess ? TQ_OK : hip_fail(ge, "decode launch");
  }
  tq::DecodeArgs a;
  a.q = q; a.q_dtype = (int32_t)dt; a.cache = (const uint8_t*)cache; a.num_blocks = num_blocks;
  a.block_tables = block_tables; a.max_blocks = max_blocks_per_seq; a.seq_lens = seq_lens;
  a.batch = batch; a.max_seq = max_seq_len; a.hkv = (int32_t)ctx->cfg.num_kv_heads; a.hq = (int32_t)ctx->cfg.num_q_heads;
  a.group = group; a.hsub = hsub; a.scale = softmax_scale;
  a.qjl_coef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / ctx->cfg.head_dim);
  a.logits = logits_out; a.out = out;
  a.counters = (uint32_t*)workspace;
  a.ws = (float*)((uint8_t*)workspace + tq::kCounterBytes);
  plan_splits(ctx->decode_wgs, batch, a.hkv * hsub, max_seq_len, &a.splits, &a.tiles_total);
  a.xcd_pairs = hsub > 1 && ((int64_t)a.splits * a.hkv * hsub * batch) % (8 * hsub) == 0;
  if ((int64_t)(a.splits + 1) * a.tiles_total >= ((int64_t)1 << 31))
    return fail(TQ_ERR_UNSUPPORTED, "max_seq_len too large");
  a.f = offsets_of(ctx->layout); a.c = ctx->consts;
  a.k_new = k_new; a.v_new = v_new;
  a.key_nc = ctx->cfg.key_mode == TQ_KEY_LLOYD_NC;
  a.klut_scale = ctx->klut_scale; a.klut_bias = ctx->klut_bias;
  if (static_scratch) {
    // the shared scratch keeps the last call's contents: zero the counters this call uses
    hipError_t ce = tq::launch_clear_words(a.counters, batch * a.hkv * hsub, stream);
    if (ce != hipSuccess) return hip_fail(ce, "scratch clear launch");
  }
  hipError_t e = tq::launch_decode(a, (int)ctx->cfg.key_bits, (int)ctx->cfg.key_mode, (int)ctx->cfg.val_bits,
                                   (int)ctx->cfg.val_mode, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return TQ_OK;
}

}  // namespace

tq_status tq_decode_attention(tq_ctx* ctx, const void* q, tq_dtype dt, const void* cache, int64_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t batch, int32_t max_seq_len, float softmax_scale, float* out,
                              float* logits_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(ctx, q, dt, cache, num_blocks, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                       softmax_scale, out, logits_out, workspace, workspace_bytes, nullptr, nullptr, stream);
}

tq_status tq_decode_attention_noalloc(tq_ctx* ctx, const void* q, tq_dtype dt, const void* cache, int64_t num_blocks,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                      float softmax_scale, float* out, float* logits_out, hipStream_t stream) {
  return decode_common(ctx, q, dt, cache, num_blocks, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                       softmax_scale, out, logits_out, nullptr, 0, nullptr, nullptr, stream, true);
}

tq_status tq_append_decode(tq_ctx* ctx, const void* k_new, const void* v_new, const void* q, tq_dtype dt,
                           void* cache, int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float softmax_scale,
                           float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!k_new) return fail(TQ_ERR_INVALID_ARG, "k_new is null");
  return decode_common(ctx, q, dt, cache, num_blocks, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                       softmax_scale, out, logits_out, workspace, workspace_bytes, k_new, v_new, stream);
}

namespace {

tq_status transfer(tq_ctx* ctx, bool to_host, void* cache, int64_t num_blocks, const int32_t* block_ids, int64_t n,
                   void* host, hipStream_t stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "ctx is null");
  if (n < 0 || num_blocks < 0) return fail(TQ_ERR_INVALID_ARG, "negative size");
  if (n == 0) return TQ_OK;
  if (!cache || !block_ids || !host) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(cache, 16) || !aligned(host, 16) || !aligned(block_ids, 4))
    return fail(TQ_ERR_INVALID_ARG, "cache and host buffer must be 16-byte aligned");
  const int64_t block_bytes = (int64_t)ctx->layout.page_bytes * ctx->cfg.num_kv_heads;
  if (n > ((int64_t)1 << 40) / block_bytes) return fail(TQ_ERR_UNSUPPORTED, "n too large");
  DeviceGuard g(ctx->device);
  // The kernel touches the host buffer through its device mapping: refuse memory
  // that is not pinned host memory mapped for the device.
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host) != hipSuccess || attr.type != hipMemoryTypeHost ||
      attr.devicePointer == nullptr) {
    (void)hipGetLastError();
    return fail(TQ_ERR_INVALID_ARG, "host buffer is not pinned host memory mapped for the device");
  }
  hipError_t e = tq::launch_transfer(to_host, cache, attr.devicePointer, block_ids, n, num_blocks, block_bytes,
                                     ctx->decode_wgs * 4, stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "transfer launch");
}

}  // namespace

tq_status tq_offload_blocks(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int32_t* block_ids, int64_t n,
                            void* host_dst, hipStream_t stream) {
  return transfer(ctx, true, const_cast<void*>(cache), num_blocks, block_ids, n, host_dst, stream);
}

tq_status tq_restore_blocks(tq_ctx* ctx, const void* host_src, const int32_t* block_ids, int64_t n, void* cache,
                            int64_t num_blocks, hipStream_t stream) {
  return transfer(ctx, false, cache, num_blocks, block_ids, n, const_cast<void*>(host_src), stream);
}

tq_status tq_dequantize_rows(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int64_t* slots, int64_t n,
                             const int64_t* rows, void* k_buf, void* v_buf, int64_t buf_rows, tq_dtype out_dt,
                             hipStream_t stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "ctx is null");
  if (n < 0 || num_blocks < 0 || buf_rows < 0) return fail(TQ_ERR_INVALID_ARG, "negative size");
  if (out_dt != TQ_F32 && out_dt != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "output dtype must be TQ_F32 or TQ_BF16");
  if (n == 0 || buf_rows == 0) return TQ_OK;
  if (!cache || !slots || !k_buf || !v_buf) return fail(TQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(cache, 16) || !aligned(k_buf, 16) || !aligned(v_buf, 16) || !aligned(slots, 8) ||
      (rows && !aligned(rows, 8)))
    return fail(TQ_ERR_INVALID_ARG, "cache and buffers must be 16-byte aligned, slots and rows 8-byte aligned");
  if ((n + 15) / 16 * (int64_t)ctx->cfg.num_kv_heads >= (int64_t(1) << 32))
    return fail(TQ_ERR_INVALID_ARG, "n too large for one launch (below 2^36 / num_kv_heads entries)");
  DeviceGuard g(ctx->device);
  if (ctx->generic) {
    tq::GenDequantArgs ga;
    std::memset(&ga, 0, sizeof ga);
    ga.cache = (const uint8_t*)cache; ga.num_blocks = num_blocks; ga.slots = slots; ga.rows = rows; ga.n = n;
    ga.buf_rows = buf_rows; ga.hkv = (int32_t)ctx->cfg.num_kv_heads;
    ga.key_bits = (int32_t)ctx->cfg.key_bits; ga.key_mode = gen_key_mode(ctx->cfg);
    ga.val_bits = (int32_t)ctx->cfg.val_bits; ga.val_mode = ctx->cfg.val_mode == TQ_VAL_LLOYD ? 1 : 0;
    ga.k_out = k_buf; ga.v_out = v_buf; ga.bf16_out = out_dt == TQ_BF16;
    ga.f = offsets_of(ctx->layout); ga.rows_b = gen_rows(ctx->layout); ga.c = ctx->gconsts;
    hipError_t ge = tq::launch_gen_dequant(ga, (int)ctx->cfg.head_dim, ctx->page_wgs, stream);
    return ge == hipSuccess ? TQ_OK : hip_fail(ge, "dequantize launch");
  }
  tq::DequantArgs a;
  for (int i = 0; i < 4; ++i) a.sign_bits[i] = ctx->sign_bits[i];
  a.cache = (const uint8_t*)cache; a.num_blocks = num_blocks; a.slots = slots; a.rows = rows; a.n = n;
  a.buf_rows = buf_rows; a.hkv = (int32_t)ctx->cfg.num_kv_heads; a.k_out = k_buf; a.v_out = v_buf;
  a.f = offsets_of(ctx->layout); a.c = ctx->consts;
  hipError_t e = tq::launch_dequant(a, (int)ctx->cfg.key_bits, (int)ctx->cfg.key_mode, (int)ctx->cfg.val_bits, (int)ctx->cfg.val_mode,
                                    out_dt == TQ_BF16, stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "dequantize launch");
}

tq_status tq_dequantize(tq_ctx* ctx, const void* cache, int64_t num_blocks, const int64_t* slots, int64_t n,
                        float* k_out, float* v_out, hipStream_t stream) {
  return tq_dequantize_rows(ctx, cache, num_blocks, slots, n, nullptr, k_out, v_out, n, TQ_F32, stream);
}

}  // extern "C"
