"""fp64 CPU oracle for TurboQuant-style KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  The product library never
routes through it and shares no code, tables or helpers with it.

Everything here is plain NumPy in float64, written for a reader to check by eye
against the pages.  Library primitives (matmul, packbits, erfc) serve as single
steps; code assignment is spelled out as a count of thresholds.

Sources (cited by page and section):
  [P1] issoh.co.jp, "TurboQuantとは？vLLM・Ollama・LM Studioの対応状況と使い方",
       sections "第1段：ランダム回転とLloyd-Max量子化" (stage 1),
       "第2段：QJLの1ビット残差と…" (stage 2, the `_nc` norm correction),
       "llama.cpp本家の専用型未採用とHadamard回転の導入" (Hadamard rotation),
       "フォーク版llama.cppのturbo3／turbo4設定" (codebook / norm separation).
  [P2] ai-navigate-news, turboquant-vllm write-up, section "Bugs Nobody Else
       Has Found" (fp32 norms; fp16 norms fail near 11k tokens).
  [P3] lilting.ch, TurboQuant article, sections "QJL: Johnson-Lindenstrauss変換で
       残差を1ビット補正する" and "TurboQuantの2段階パイプライン".
  [P4] qiita, AMD 4-bit KV caching in LMCache, sections "4bitという名前だけでは…"
       (two 4-bit codes per uint8) and "小さな保存・復元コードで…" (byte example).

Readings taken where the pages are silent:
  R1  rotation y = H (s * x) / sqrt(d), Sylvester H in natural order, signs first.
  R2  codebook = Lloyd-Max for N(0, 1/d), solved on the positive half and mirrored.
  R5  norm correction: stored norm = ||k|| / ||C[code]||, so ||k_hat|| = ||k||.
  R6  zero key: codes = 2^(b-1), stored norm 0.
  R11 uniform values: scale = fl32((max-min)/(2^b-1)) (the stored fp32 scale),
      code = rint((v-min)/scale) of the exact quotient, round half to even.
  R18 decision bands (coordinates this close to a boundary may take either code):
      keys: min_j |y_i - t_j| with y on the unit sphere; uniform values:
      |frac(x) - 1/2| / (2^b - 1) in [0, 1] range units; QJL signs: the cosine
      |(S r')_i| / (||S_i|| ||r'||); PolarQuant angles: radians to the nearest
      cell edge (level 1 wraps at +-pi).
  R12 bit order: LSB-first stream per vector (generalises [P4]'s nibble order).
  R13 QJL: residual in the rotated frame, m = d rows, sign(0) -> bit 1.
  R14 GQA: q head h reads kv head h // (Hq/Hkv); softmax scale supplied by caller.
  R26 PolarQuant keys ([P3] PolarQuant section): after the stage-1 rotation the
      vector goes through the recursive polar transform (pairs -> radius and
      angle, radii paired again, down to one radius and d-1 angles); every angle
      takes a b-bit uniform grid over its range (level 1: [-pi, pi), higher
      levels: [0, pi/2]) with cell-centre reconstruction; the radius is fp32
      (R7).  Stream order of the 128 slots: subtree-major (R27).
  R24 FP8 keys ([P1] preset table: the k8v4 preset stores keys in FP8, 2.6x):
      OCP E4M3 of each raw key coordinate (no rotation, no per-token scale),
      nearest value with ties to the even code, magnitudes above 448 saturate.

Readings no page fixes (conventions; each function is pinned to mathematics,
not to a page): the norm-correction definition (R5: the reconstruction keeps
the key's norm), the toy workload's Lloyd-Max values (the key quantizer's
pins), the QJL frame and m (R13: unbiased, closed-form variance), the 2- and
3-bit bit order (R12: exhaustive pack/unpack, the page's 4-bit bytes).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

BLOCK_TOKENS = 16
FORMAT_VERSION = 2


# ----------------------------------------------------------------------------
# Rotation  [P1 stage 1; P1 Hadamard rotation section]
# ----------------------------------------------------------------------------
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (entries +-1, natural order) as int64.

    H_1 = [1];  H_2n = [[H_n, H_n], [H_n, -H_n]].  Built as a dense matrix, not a
    butterfly, so it checks the GPU's butterfly independently.
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs: np.ndarray) -> np.ndarray:
    """R = H diag(s) / sqrt(d): random signs first, then the normalized WHT (R1)."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return hadamard(d).astype(np.float64) * s[None, :] / math.sqrt(d)


# ----------------------------------------------------------------------------
# Lloyd-Max codebook  [P1 stage 1: per-coordinate Lloyd-Max; calibration-free]
# ----------------------------------------------------------------------------
def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x):
    """P(Z > x) for standard normal Z, accurate in the tail."""
    return 0.5 * np.array([math.erfc(v / math.sqrt(2.0)) if np.isfinite(v) else (0.0 if v > 0 else 1.0)
                           for v in np.atleast_1d(x)])


def lloyd_max_standard_normal(bits: int, tol: float = 1e-15, max_iter: int = 2_000_000
                              ) -> Tuple[np.ndarray, np.ndarray]:
    """Lloyd-Max quantizer of N(0,1) with 2^bits levels (float64).

    Alternates the two optimality conditions until the centroids stop moving:
      thresholds are midpoints of neighbouring centroids;
      each centroid is the conditional mean of its cell:
        c = (phi(a) - phi(b)) / (P(Z > a) - P(Z > b)).
    Solved on the positive half (the density is symmetric and log-concave, so
    the fixpoint is unique and symmetric), then mirrored.
    Returns (centroids ascending [2^b], thresholds ascending [2^b - 1]).
    """
    k = 1 << (bits - 1)                      # positive centroids
    # start at the conditional means of equal-probability cells
    probs = 0.5 + 0.5 * (np.arange(k + 1) / k)
    from statistics import NormalDist
    edges = np.array([NormalDist().inv_cdf(min(p, 1 - 1e-12)) for p in probs])
    edges[0], edges[-1] = 0.0, np.inf
    c = np.empty(k)
    for i in range(k):
        a, b = edges[i], edges[i + 1]
        c[i] = (_phi(a) - (0.0 if np.isinf(b) else _phi(b))) / (_upper_tail(a)[0] - _upper_tail(b)[0])
    # With many levels the alternation converges slowly (its error contracts by
    # about 1 - O(1/k^2) per round); from 5 bits on a bounded number of rounds is
    # followed by Newton's method on the same fixpoint equations.
    rounds = max_iter if bits <= 4 else 2000
    for _ in range(rounds):
        t = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]])
        upper = _upper_tail(t)
        dens = _phi(t[:-1]) - _phi(t[1:])          # phi(inf) = 0
        c_new = dens / (upper[:-1] - upper[1:])
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            break
    if bits > 4:
        c = _lloyd_newton(c, tol)
    pos_t = 0.5 * (c[:-1] + c[1:])
    centroids = np.concatenate([-c[::-1], c])
    thresholds = np.concatenate([-pos_t[::-1], [0.0], pos_t])
    return centroids, thresholds


def _lloyd_newton(c: np.ndarray, tol: float, max_steps: int = 60) -> np.ndarray:
    """Newton's method on G(c) = c - m(c) = 0 for the positive centroids c, where
    m_i is the mean of N(0,1) on the cell (a_i, b_i) whose edges are the midpoints
    a_i = (c_{i-1} + c_i)/2 (a_0 = 0) and b_i = (c_i + c_{i+1})/2 (last b = inf).
    The mean of a cell moves with its edges as dm/da = phi(a)(m - a)/P and
    dm/db = phi(b)(b - m)/P (P = the cell's mass), so the Jacobian of G is
    tridiagonal."""
    k = c.shape[0]
    for _ in range(max_steps):
        t = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]])
        a, b = t[:-1], t[1:]
        upper = _upper_tail(t)
        P = upper[:-1] - upper[1:]
        m = (_phi(a) - _phi(b)) / P
        G = c - m
        dA = _phi(a) * (m - a) / P
        dA[0] = 0.0                                 # a_0 = 0 does not move
        dB = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)) * (b - m) / P)
        J = np.zeros((k, k))
        idx = np.arange(k)
        J[idx, idx] = 1.0 - 0.5 * dA - 0.5 * dB
        J[idx[1:], idx[1:] - 1] = -0.5 * dA[1:]
        J[idx[:-1], idx[:-1] + 1] = -0.5 * dB[:-1]
        delta = np.linalg.solve(J, G)
        c = c - delta
        if np.max(np.abs(delta)) < tol:
            break
    return c


@dataclasses.dataclass(frozen=True)
class Codebook:
    bits: int
    centroids: np.ndarray    # float64 [2^b], ascending
    thresholds: np.ndarray   # float64 [2^b - 1], ascending


def codebook(bits: int, d: int) -> Codebook:
    """Lloyd-Max codebook for one rotated unit-vector coordinate, modelled N(0, 1/d) (R2)."""
    c, t = lloyd_max_standard_normal(bits)
    s = 1.0 / math.sqrt(d)
    return Codebook(bits, c * s, t * s)


def assign_codes(y: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """code = #{j : t_j <= y} for every coordinate (cells are [t_{j-1}, t_j))."""
    return (y[..., None] >= thresholds).sum(axis=-1).astype(np.int64)


def boundary_distance(y: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """min_j |y - t_j|: distance of each rotated coordinate to a decision boundary."""
    return np.abs(y[..., None] - thresholds).min(axis=-1)


def fl32(x):
    """Round float64 values to the nearest float32 (the stored precision) and widen back."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Keys: norm separation, rotation, Lloyd-Max codes, norm correction, QJL
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class KeyCodes:
    codes: np.ndarray        # int64 [..., d]
    norm: np.ndarray         # float64 [...]  stored scalar, already rounded to fp32
    y: np.ndarray            # float64 [..., d] rotated unit vector (diagnostics / band)
    band: np.ndarray         # float64 [..., d] distance to the nearest threshold
    qjl_bits: Optional[np.ndarray] = None   # int64 [..., m] 1 if (S r')_i >= 0
    qjl_norm: Optional[np.ndarray] = None   # float64 [...] ||r'||, rounded to fp32
    qjl_band: Optional[np.ndarray] = None   # float64 [..., m] |(S r')_i| / (||S_i|| ||r'||)


def quantize_keys(k: np.ndarray, signs: np.ndarray, cb: Codebook, mode: str,
                  S: Optional[np.ndarray] = None) -> KeyCodes:
    """Stage 1 (and optionally stage 2) key quantization of vectors k[..., d].

    [P1 stage 1] random rotation then per-coordinate Lloyd-Max on the unit vector;
    [P1 fork section; P2 bugs section] norm kept apart from the codes, in fp32;
    [P1 stage 2] `_nc` = norm correction (definition R5);
    [P3 QJL section] 1-bit signs of a Gaussian projection of the residual.
    mode: "lloyd" (plain norm), "lloyd_nc" (corrected norm), "lloyd_qjl" (plain + QJL).
    """
    if mode == "fp8":
        return quantize_keys_fp8(k)
    if mode == "polar":
        return quantize_keys_polar(k, signs, cb.bits)
    k = np.asarray(k, dtype=np.float64)
    R = rotation_matrix(signs)
    n = np.sqrt((k * k).sum(axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = k / safe[..., None]
    y = u @ R.T                                   # y = R u  (row vectors)
    y = np.where((n > 0)[..., None], y, 0.0)      # zero key -> y = 0 (R6)
    codes = assign_codes(y, cb.thresholds)
    chat = cb.centroids[codes]
    if mode == "lloyd_nc":
        cn = np.sqrt((chat * chat).sum(axis=-1))
        norm = fl32(n / cn)
    elif mode in ("lloyd", "lloyd_qjl"):
        norm = fl32(n)
    else:
        raise ValueError(mode)
    out = KeyCodes(codes=codes, norm=norm, y=y, band=boundary_distance(y, cb.thresholds))
    if mode == "lloyd_qjl":
        if S is None:
            raise ValueError("QJL needs S")
        S = np.asarray(S, dtype=np.float64)
        r = n[..., None] * y - norm[..., None] * chat          # residual, rotated frame (R13)
        z = r @ S.T
        out.qjl_bits = (z >= 0).astype(np.int64)
        rn = np.sqrt((r * r).sum(axis=-1))
        out.qjl_norm = fl32(rn)
        srow = np.sqrt((S * S).sum(axis=1))
        out.qjl_band = np.abs(z) / (srow * np.where(rn > 0, rn, 1.0)[..., None])
    return out


def dequantize_keys(codes: np.ndarray, norm: np.ndarray, signs: np.ndarray, cb: Codebook) -> np.ndarray:
    """Stage-1 reconstruction in the original basis: k_hat = norm * R^T C[code]."""
    R = rotation_matrix(signs)
    return np.asarray(norm, dtype=np.float64)[..., None] * (cb.centroids[codes] @ R)


# ----------------------------------------------------------------------------
# FP8 keys  [P1 preset table: one serving preset keeps the keys in FP8 and the
# values in 4 bits]  (R24)
# ----------------------------------------------------------------------------
FP8_MAX = 448.0


def fp8_e4m3_value(code) -> np.ndarray:
    """Value of E4M3 bytes: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent 0 holds the subnormals m * 2^-9; there are no infinities and
    S.1111.111 is NaN."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((code & 0x7F) == 0x7F, np.nan, sign * mag)


def quantize_fp8_e4m3(x) -> np.ndarray:
    """E4M3 code of each value: the nearest finite value, ties to the even code
    (even mantissa), magnitudes above 448 saturating to 448; the sign bit is
    kept, so -0 and negatives that round to zero give 0x80."""
    x = np.asarray(x, dtype=np.float64)
    mags = fp8_e4m3_value(np.arange(0x7F))           # codes 0..126, increasing
    a = np.minimum(np.abs(x), FP8_MAX)
    hi = np.minimum(np.searchsorted(mags, a, side="left"), 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return code | np.where(np.signbit(x), 0x80, 0)


def quantize_keys_fp8(k: np.ndarray) -> KeyCodes:
    """FP8 keys: codes are the E4M3 bytes of the coordinates; nothing else is
    stored (norm 1 stands for 'no scale').  The decision is exact on both sides,
    so there is no boundary band (inf)."""
    k = np.asarray(k, dtype=np.float64)
    return KeyCodes(codes=quantize_fp8_e4m3(k), norm=np.ones(k.shape[:-1]), y=k,
                    band=np.full(k.shape, np.inf))


# ----------------------------------------------------------------------------
# PolarQuant keys  [P3 PolarQuant section: recursive polar transform, one
# radius and d-1 angles, angles on a uniform grid with no per-block constants]
# (R26, R27)
# ----------------------------------------------------------------------------
def polar_slot_map(d: int = 128):
    """(level, node) stored in each of the d code slots; (0, 0) is padding.

    Quarter g of the coordinates (32g .. 32g+31 at d = 128) owns slots 32g..32g+31:
    its 16 level-1 angles, 8 level-2, 4 level-3, 2 level-4 and 1 level-5 angle,
    in node order; slot 32g+31 holds the root (g = 0), the two level-6 angles
    (g = 1, 2) or padding (g = 3)."""
    assert d == 128
    slots = []
    for g in range(4):
        for level, count in ((1, 16), (2, 8), (3, 4), (4, 2), (5, 1)):
            slots += [(level, count * g + i) for i in range(count)]
        slots.append({0: (7, 0), 1: (6, 0), 2: (6, 1), 3: (0, 0)}[g])
    return slots


def polar_forward(y: np.ndarray):
    """Recursive polar transform of y[..., d]: angles per level (level 1: atan2 of
    coordinate pairs; level l > 1: atan2 of pairs of level l-1 radii) and the
    final radius ||y||."""
    rho = np.asarray(y, dtype=np.float64)
    angles = {}
    level = 1
    while rho.shape[-1] > 1:
        a, b = rho[..., 0::2], rho[..., 1::2]
        angles[level] = np.arctan2(b, a)
        rho = np.hypot(a, b)
        level += 1
    return angles, rho[..., 0]


def polar_inverse(angles: dict, radius) -> np.ndarray:
    """Inverse transform: top down, a node of radius r and angle t gives its
    children r cos t and r sin t."""
    rho = np.asarray(radius, dtype=np.float64)[..., None]
    for level in sorted(angles, reverse=True):
        t = angles[level]
        rho = np.stack([rho * np.cos(t), rho * np.sin(t)], axis=-1).reshape(t.shape[:-1] + (2 * t.shape[-1],))
    return rho


def polar_grid(level: int, bits: int):
    """(lowest edge, cell width) of the uniform angle grid of a level."""
    return (-math.pi, 2 * math.pi / (1 << bits)) if level == 1 else (0.0, (math.pi / 2) / (1 << bits))


def polar_codes(theta: np.ndarray, level: int, bits: int):
    """Cell index of each angle (level 1 wraps around: pi is -pi) and its distance to
    the nearest cell edge (the decision boundaries)."""
    lo, w = polar_grid(level, bits)
    x = (theta - lo) / w
    if level == 1:
        code = np.floor(x).astype(np.int64) % (1 << bits)
        band = np.abs(x - np.rint(x)) * w
    else:
        code = np.clip(np.floor(x), 0, (1 << bits) - 1).astype(np.int64)
        inner = np.clip(np.rint(x), 1, (1 << bits) - 1)      # edges between cells
        band = np.abs(x - inner) * w
    return code, band


def polar_angle(code, level: int, bits: int) -> np.ndarray:
    lo, w = polar_grid(level, bits)
    return lo + (np.asarray(code, dtype=np.float64) + 0.5) * w


def quantize_keys_polar(k: np.ndarray, signs: np.ndarray, bits: int) -> KeyCodes:
    """PolarQuant keys: y = R k, polar transform of y, b-bit angle codes in slot
    order; stored scalar = fp32 radius (= ||k||).  An angle whose pair has zero
    radius is undefined and counted in the band."""
    k = np.asarray(k, dtype=np.float64)
    y = k @ rotation_matrix(signs).T
    angles, radius = polar_forward(y)
    # radii below each angle (to flag undefined angles)
    rho = y
    node_r = {}
    level = 1
    while rho.shape[-1] > 1:
        a, b = rho[..., 0::2], rho[..., 1::2]
        rho = np.hypot(a, b)
        node_r[level] = rho
        level += 1
    slots = polar_slot_map(k.shape[-1])
    codes = np.zeros(k.shape, dtype=np.int64)
    band = np.full(k.shape, np.inf)
    for i, (level, node) in enumerate(slots):
        if level == 0:
            continue
        c, bd = polar_codes(angles[level][..., node], level, bits)
        codes[..., i] = c
        band[..., i] = np.where(node_r[level][..., node] > 0, bd, 0.0)
    return KeyCodes(codes=codes, norm=fl32(radius), y=y, band=band)


def dequantize_keys_polar(codes: np.ndarray, norm, signs: np.ndarray, bits: int) -> np.ndarray:
    """k_hat = R^T y_hat, y_hat the inverse polar transform of the cell-centre angles
    and the stored radius."""
    codes = np.asarray(codes, dtype=np.int64)
    d = codes.shape[-1]
    slots = polar_slot_map(d)
    angles = {}
    for level in range(1, 8):
        angles[level] = np.zeros(codes.shape[:-1] + (d >> level,))
    for i, (level, node) in enumerate(slots):
        if level:
            angles[level][..., node] = polar_angle(codes[..., i], level, bits)
    y_hat = polar_inverse(angles, norm)
    return y_hat @ rotation_matrix(signs)


# ----------------------------------------------------------------------------
# Values  [P1 stage 2: stage 1 paired with uniform quantization of values]
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class ValueCodes:
    codes: np.ndarray
    vmin: np.ndarray     # float64 [...] (fp32 value)
    scale: np.ndarray    # float64 [...] (fp32 value)
    band: np.ndarray     # float64 [..., d] |frac(x) - 1/2| / (2^b - 1)


def quantize_values_uniform(v: np.ndarray, bits: int) -> ValueCodes:
    """Per-vector uniform quantizer with fp32 min and scale (R11).

    [P1 stage 2: stage 1 pairs with uniform quantization of the values]
      min, max: exact (the inputs are bf16/fp32 values, so both are fp32 values);
      scale = fl32((max - min) / (2^b - 1)), the stored fp32 scale;
      code  = clamp(rint((v - min) / scale), 0, 2^b - 1), round half to even, the
              quotient taken exactly (fp64 holds it to far below the band) with
              the stored min and scale.
    For bf16 inputs max - min is an fp32 value, and an fp64 quotient of fp32
    values rounds to the correctly rounded fp32 quotient (53 >= 2*24 + 2 bits, so
    the double rounding is innocuous).
    A constant vector has scale 0 and all codes 0.  The band is the quotient's
    distance to a rounding boundary in [0, 1] range units: |frac(x) - 1/2| / (2^b - 1).
    """
    v64 = np.asarray(v, dtype=np.float64)
    levels = (1 << bits) - 1
    mn = v64.min(axis=-1)
    mx = v64.max(axis=-1)
    sc = fl32((mx - mn) / levels)
    safe = np.where(sc > 0, sc, 1.0)
    x = (v64 - mn[..., None]) / safe[..., None]
    x = np.where((sc > 0)[..., None], x, 0.0)
    codes = np.clip(np.rint(x), 0, levels).astype(np.int64)
    band = np.abs(x - np.floor(x) - 0.5) / levels
    band = np.where((sc > 0)[..., None], band, np.inf)
    return ValueCodes(codes=codes, vmin=mn, scale=sc, band=band)


def dequantize_values_uniform(codes, vmin, scale) -> np.ndarray:
    return np.asarray(vmin, np.float64)[..., None] + np.asarray(scale, np.float64)[..., None] * codes


# ----------------------------------------------------------------------------
# Bit packing  [P4: two 4-bit codes per byte, element 2i in the low nibble] (R12)
# ----------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bit stream per vector: code i fills stream bits [b*i, b*i+b),
    stream bit k is bit (k mod 8) of byte k // 8.  codes[..., n] -> uint8[..., n*b/8]."""
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.shape[-1]
    if (n * bits) % 8:
        raise ValueError("vector does not fill whole bytes")
    bitplanes = (codes[..., None] >> np.arange(bits)) & 1          # [..., n, b], LSB first
    stream = bitplanes.reshape(codes.shape[:-1] + (n * bits,)).astype(np.uint8)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_codes(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    stream = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1, bitorder="little")
    stream = stream[..., : n * bits].reshape(packed.shape[:-1] + (n, bits)).astype(np.int64)
    return (stream << np.arange(bits)).sum(axis=-1)


# ----------------------------------------------------------------------------
# Paged cache format (format version 2).  A page holds 16 tokens of one KV head;
# fields are stored one after another, each holding one row per token slot:
#   key codes, key norm (f32; absent for FP8 keys), [QJL sign bits, QJL residual norm (f32)],
#   value codes, value min or value norm (f32), [value scale (f32)].
# Every field is slot-major (row of slot s at field + s * row_bytes) except the
# value codes, which are plane-major: byte p of slot s's row sits at
# field + 16 * p + s (the 16 slots of one byte position are contiguous).
# The cache is [num_blocks][num_kv_heads][page_bytes]; slot = block*16 + offset.
# [P4 transfer section: the reader must know the format id/version and layout]
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    head_dim: int
    num_kv_heads: int
    num_q_heads: int
    key_bits: int
    key_mode: str       # "lloyd" | "lloyd_nc" | "lloyd_qjl" | "fp8" (key_bits 8) | "polar"
    val_bits: int
    val_mode: str       # "uniform" | "lloyd"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def page_fields(cfg: Config) -> Dict[str, Tuple[int, int]]:
    """Byte offset and per-token row size of every field inside one page."""
    d = cfg.head_dim
    rows = [("kcodes", d * cfg.key_bits // 8)]
    if cfg.key_mode != "fp8":
        rows += [("knorm", 4)]
    if cfg.key_mode == "lloyd_qjl":
        rows += [("ksigns", d // 8), ("kres", 4)]
    rows += [("vcodes", d * cfg.val_bits // 8)]
    rows += [("vmin", 4), ("vscale", 4)] if cfg.val_mode == "uniform" else [("vnorm", 4)]
    out, off = {}, 0
    for name, size in rows:
        out[name] = (off, size)
        off += BLOCK_TOKENS * size
    out["_page"] = (off, 0)
    return out


def page_bytes(cfg: Config) -> int:
    return page_fields(cfg)["_page"][0]


def new_cache(cfg: Config, num_blocks: int, fill: int = 0xA5) -> np.ndarray:
    return np.full((num_blocks, cfg.num_kv_heads, page_bytes(cfg)), fill, dtype=np.uint8)


def _f32_bytes(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype("<f4").view(np.uint8).reshape(np.shape(x) + (4,))


def _bytes_f32(b) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint8).view("<f4")[..., 0].astype(np.float64)


@dataclasses.dataclass
class Quantized:
    """All stored fields of a batch of token-heads, shape [N, Hkv, ...]."""
    key: KeyCodes
    val_codes: np.ndarray
    val_a: np.ndarray          # value min (uniform) or value norm (lloyd)
    val_b: Optional[np.ndarray]  # value scale (uniform)
    val_band: np.ndarray


def quantize_tokens(cfg: Config, k, v, signs, kcb: Codebook, vcb: Optional[Codebook],
                    S=None) -> Quantized:
    """Quantize N new tokens' keys and values [N, Hkv, d] (one pass per token: the
    method is online, past tokens are never revisited) [P3 pipeline section]."""
    kq = quantize_keys(k, signs, kcb, cfg.key_mode, S)
    if cfg.val_mode == "uniform":
        vq = quantize_values_uniform(v, cfg.val_bits)
        return Quantized(kq, vq.codes, vq.vmin, vq.scale, vq.band)
    vk = quantize_keys(v, signs, vcb, "lloyd")
    return Quantized(kq, vk.codes, vk.norm, None, vk.band)


def write_tokens(cfg: Config, cache: np.ndarray, slots: np.ndarray, qz: Quantized) -> None:
    """Store every field of N token-heads at slot (block*16 + offset) of each KV head."""
    f = page_fields(cfg)
    slots = np.asarray(slots, dtype=np.int64)
    blk, off = slots // BLOCK_TOKENS, slots % BLOCK_TOKENS
    rows = {
        "kcodes": pack_codes(qz.key.codes, cfg.key_bits),
        "vcodes": pack_codes(qz.val_codes, cfg.val_bits),
    }
    if cfg.key_mode != "fp8":
        rows["knorm"] = _f32_bytes(qz.key.norm)
    if cfg.key_mode == "lloyd_qjl":
        rows["ksigns"] = pack_codes(qz.key.qjl_bits, 1)
        rows["kres"] = _f32_bytes(qz.key.qjl_norm)
    if cfg.val_mode == "uniform":
        rows["vmin"] = _f32_bytes(qz.val_a)
        rows["vscale"] = _f32_bytes(qz.val_b)
    else:
        rows["vnorm"] = _f32_bytes(qz.val_a)
    for name, data in rows.items():
        base, size = f[name]
        for i in range(slots.shape[0]):
            for h in range(cfg.num_kv_heads):
                if name == "vcodes":
                    cache[blk[i], h, base + BLOCK_TOKENS * np.arange(size) + off[i]] = data[i, h]
                else:
                    start = base + off[i] * size
                    cache[blk[i], h, start:start + size] = data[i, h]


def read_tokens(cfg: Config, cache: np.ndarray, slots: np.ndarray, head: int) -> Dict[str, np.ndarray]:
    """Parse the stored fields of the given slots of one KV head."""
    f = page_fields(cfg)
    slots = np.asarray(slots, dtype=np.int64)
    blk, off = slots // BLOCK_TOKENS, slots % BLOCK_TOKENS
    out = {}
    for name, (base, size) in f.items():
        if name == "_page":
            continue
        if name == "vcodes":
            idx = base + off[:, None] + BLOCK_TOKENS * np.arange(size)[None, :]
        else:
            idx = base + off[:, None] * size + np.arange(size)[None, :]
        raw = cache[blk[:, None], head, idx]
        if name == "kcodes":
            out[name] = unpack_codes(raw, cfg.key_bits, cfg.head_dim)
        elif name == "vcodes":
            out[name] = unpack_codes(raw, cfg.val_bits, cfg.head_dim)
        elif name == "ksigns":
            out[name] = unpack_codes(raw, 1, cfg.head_dim)
        else:
            out[name] = _bytes_f32(raw)
    return out


def quantize_append(cfg: Config, cache, k, v, slots, signs, kcb, vcb=None, S=None) -> Quantized:
    qz = quantize_tokens(cfg, k, v, signs, kcb, vcb, S)
    write_tokens(cfg, cache, slots, qz)
    return qz


# ----------------------------------------------------------------------------
# Decode attention over the packed cache  [P1 zero-loss section: logits are what
# the 8x figure measures; P2: a fused attention is needed; P3 QJL section]
# ----------------------------------------------------------------------------
def dequantize_slots(cfg: Config, cache, slots, head: int, signs, kcb: Codebook,
                     vcb: Optional[Codebook]) -> Tuple[np.ndarray, np.ndarray, Dict[str, np.ndarray]]:
    """k_hat (stage 1) and v_hat [n, d] in the original basis for the given slots of one head."""
    f = read_tokens(cfg, cache, slots, head)
    if cfg.key_mode == "fp8":
        k_hat = fp8_e4m3_value(f["kcodes"])
    elif cfg.key_mode == "polar":
        k_hat = dequantize_keys_polar(f["kcodes"], f["knorm"], signs, cfg.key_bits)
    else:
        k_hat = dequantize_keys(f["kcodes"], f["knorm"], signs, kcb)
    if cfg.val_mode == "uniform":
        v_hat = dequantize_values_uniform(f["vcodes"], f["vmin"], f["vscale"])
    else:
        v_hat = dequantize_keys(f["vcodes"], f["vnorm"], signs, vcb)
    return k_hat, v_hat, f


def qjl_correction(q: np.ndarray, signs, S, fields) -> np.ndarray:
    """Second-stage estimate of <q, r> for every token: ||r'|| sqrt(pi/2)/m <S R q, 2 sigma - 1>.

    For g ~ N(0, I): E[(g.a) sign(g.b)] = sqrt(2/pi) (a.b)/||b||, which makes the
    sum over the m rows of S an unbiased estimate of <R q, r'> = <q, r>.
    """
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    p = S @ (rotation_matrix(signs) @ np.asarray(q, np.float64))
    pm = 2.0 * fields["ksigns"] - 1.0
    return fields["kres"] * math.sqrt(math.pi / 2.0) / m * (pm @ p)


def attention_one(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float,
                  correction: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """logits = scale * <q, k_hat_j> (+ scale * QJL correction); out = softmax(logits) @ v_hat.

    Direct max-subtracted softmax (the definition); empty context gives zeros."""
    if k_hat.shape[0] == 0:
        return np.zeros(0), np.zeros(v_hat.shape[-1])
    dots = k_hat @ np.asarray(q, np.float64)
    if correction is not None:
        dots = dots + correction
    logits = scale * dots
    e = np.exp(logits - logits.max())
    p = e / e.sum()
    return logits, p @ v_hat


def decode_attention(cfg: Config, q: np.ndarray, cache, block_tables, seq_lens, scale: float,
                     signs, kcb: Codebook, vcb: Optional[Codebook] = None, S=None,
                     heads: Optional[list] = None):
    """Attention of every (sequence, q head) over its packed context.

    q: [B, Hq, d].  Returns (logits list-of-arrays per (b,h), out [B, Hq, d]).
    `heads` optionally restricts the work to a list of (b, h) pairs.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    g = cfg.group
    out = np.zeros((B, Hq, d))
    logits = {}
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    by_kv: Dict[Tuple[int, int], list] = {}
    for b, h in todo:
        by_kv.setdefault((b, h // g), []).append(h)
    for (b, kvh), hs in sorted(by_kv.items()):
        n = int(seq_lens[b])
        t = np.arange(n, dtype=np.int64)
        slots = np.asarray(block_tables[b], np.int64)[t // BLOCK_TOKENS] * BLOCK_TOKENS + t % BLOCK_TOKENS
        k_hat, v_hat, fields = dequantize_slots(cfg, cache, slots, kvh, signs, kcb, vcb)
        for h in hs:
            corr = qjl_correction(q[b, h], signs, S, fields) if cfg.key_mode == "lloyd_qjl" else None
            lg, o = attention_one(q[b, h], k_hat, v_hat, scale, corr)
            logits[(b, h)] = lg
            out[b, h] = o
    return logits, out
