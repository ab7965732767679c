"""Shared helpers of the GPU parity tests: build inputs from the seeded recipes,
run the HIP library through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np

from kv_cache_vector_randomized_amd import synth, tq
from oracle import tq_oracle as O

BAND = 1e-6          # coordinates this close to a decision boundary are excluded from bit-exact checks
REL_TOL = 1e-4       # logits and attention outputs, relative (per (sequence, q head) vector)
NORM_ULP = 2         # stored fp32 norms: within 2 ulp of the oracle's fp32 rounding
# QJL residual norm rho, from the fp32 rotation of the key (the MFMA sums and three
# butterfly levels, 7.5 u), the fp32 norm (1 u), the residual's fma (1 u) and an fp32
# sum of squares with its square root (19 u on rho), u = 2^-24:
# |rho_gpu - rho| <= 9 u ||k|| + 20 u rho
RHO_REL_K, RHO_REL_RHO = 9 * 2.0 ** -24, 20 * 2.0 ** -24

# Per-workload parity figures, written out at the end of the session (conftest.py)
REPORT: dict = {}


def report(test: str, workload: str, **fig):
    """Record parity figures of one test and workload; counts add up, maxima are kept."""
    rec = REPORT.setdefault((test, workload), {})
    for k, v in fig.items():
        if k.startswith("max_") or k.startswith("worst_"):
            rec[k] = max(rec.get(k, 0.0), float(v))
        else:
            rec[k] = rec.get(k, 0) + int(v)


def ulp_distance(a, b) -> np.ndarray:
    """Distance in fp32 ulps between non-negative fp32 values (float arrays)."""
    ia = np.asarray(a, np.float64).astype(np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float64).astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def elem_err(a, b) -> float:
    """Largest elementwise error relative to the largest reference magnitude."""
    m = np.max(np.abs(b)) if np.size(b) else 0.0
    d = np.max(np.abs(a - b)) if np.size(b) else 0.0
    return d / m if m > 0 else d


def oracle_config(w: synth.Workload) -> O.Config:
    return O.Config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.key_bits, w.key_mode, w.val_bits, w.val_mode)


def lib_config(w: synth.Workload) -> tq.Config:
    return tq.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.key_bits, w.key_mode, w.val_bits,
                          w.val_mode)


def qjl_S(w):
    return synth.qjl_matrix(w.head_dim) if w.key_mode == "lloyd_qjl" else None


def signs(w):
    return synth.sign_vector(w.seed, w.head_dim)


def make_context(w):
    return tq.Context(lib_config(w), signs(w), qjl_S(w))


def oracle_codebooks(w):
    kcb = O.codebook(w.key_bits, w.head_dim) if w.key_mode != "fp8" else None   # FP8 keys have none
    vcb = O.codebook(w.val_bits, w.head_dim) if w.val_mode == "lloyd" else None
    return kcb, vcb


def as_f64(x, w):
    return (synth.bf16_bits_to_f32(x) if w.dtype == "bf16" else np.asarray(x, np.float32)).astype(np.float64)


def upload(x, w, torch):
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def oracle_quantize(w, k, v):
    kcb, vcb = oracle_codebooks(w)
    S = qjl_S(w)
    return O.quantize_tokens(oracle_config(w), as_f64(k, w), as_f64(v, w), signs(w), kcb, vcb,
                             None if S is None else S.astype(np.float64))


def written_mask(cfg: O.Config, shape, slots):
    """Bytes of the cache that a write of `slots` may touch."""
    f = O.page_fields(cfg)
    m = np.zeros(shape, bool)
    for s in np.asarray(slots, np.int64):
        if s < 0 or s >= shape[0] * 16:
            continue
        for name, (base, size) in f.items():
            if name == "vcodes":
                m[s // 16, :, base + (s % 16) + 16 * np.arange(size)] = True
            elif name != "_page":
                m[s // 16, :, base + (s % 16) * size: base + (s % 16 + 1) * size] = True
    return m


def compare_append(w, gpu_cache: np.ndarray, slots, qz: O.Quantized, report: dict):
    """GPU-written fields vs the oracle's: codes bit-exact outside the boundary band (inside it the
    code may be either neighbour), fp32 scalars within their rounding tolerance."""
    cfg = oracle_config(w)
    slots = np.asarray(slots, np.int64)
    for h in range(cfg.num_kv_heads):
        f = O.read_tokens(cfg, gpu_cache, slots, h)
        kc, kref = f["kcodes"], qz.key.codes[:, h]
        band = qz.key.band[:, h] < BAND
        diff = kc != kref
        assert not np.any(diff & ~band), f"key code mismatch outside the band (head {h})"
        if cfg.key_mode == "polar":     # level-1 angles wrap around: neighbours modulo 2^b
            assert np.all(np.isin((kc - kref) % (1 << cfg.key_bits), [0, 1, (1 << cfg.key_bits) - 1]))
        else:
            assert np.all(np.abs(kc - kref) <= 1)
        report["key_band"] = report.get("key_band", 0) + int(band.sum())
        report["key_band_flips"] = report.get("key_band_flips", 0) + int(diff.sum())
        clean = ~diff.any(axis=1)
        if cfg.key_mode != "fp8":        # FP8 keys store no norm
            # the corrected norm depends on the codes: rows with a band flip are skipped there
            rows = clean if cfg.key_mode == "lloyd_nc" else np.ones_like(clean)
            u = ulp_distance(f["knorm"], qz.key.norm[:, h])[rows]
            assert np.all(u <= NORM_ULP), u.max()
            report["max_knorm_ulp"] = max(report.get("max_knorm_ulp", 0), int(u.max()) if u.size else 0)
        if cfg.key_mode == "lloyd_qjl":
            sband = qz.key.qjl_band[:, h] < BAND
            sdiff = f["ksigns"] != qz.key.qjl_bits[:, h]
            assert not np.any(sdiff[clean] & ~sband[clean]), "QJL sign mismatch outside the band"
            report["sign_band"] = report.get("sign_band", 0) + int(sband.sum())
            report["sign_band_flips"] = report.get("sign_band_flips", 0) + int(sdiff[clean].sum())
            rho, n = qz.key.qjl_norm[:, h], qz.key.norm[:, h]
            dr = np.abs(f["kres"] - rho)
            assert np.all((dr <= RHO_REL_K * n + RHO_REL_RHO * rho)[clean]), (dr / (n + rho))[clean].max()
            rel = (dr / np.maximum(n, 1e-30))[clean]
            report["max_rho_err_over_knorm"] = max(report.get("max_rho_err_over_knorm", 0.0),
                                                   float(rel.max()) if rel.size else 0.0)
        vc, vref = f["vcodes"], qz.val_codes[:, h]
        vband = qz.val_band[:, h] < BAND
        vdiff = vc != vref
        assert not np.any(vdiff & ~vband), f"value code mismatch outside the band (head {h})"
        assert np.all(np.abs(vc - vref) <= 1)
        report["val_band"] = report.get("val_band", 0) + int(vband.sum())
        report["val_band_flips"] = report.get("val_band_flips", 0) + int(vdiff.sum())
        if cfg.val_mode == "uniform":
            assert np.array_equal(f["vmin"], qz.val_a[:, h])
            if w.dtype == "bf16":
                assert np.array_equal(f["vscale"], qz.val_b[:, h])   # correctly rounded division
            else:
                assert np.allclose(f["vscale"], qz.val_b[:, h], rtol=2 ** -23, atol=0)
        else:
            u = ulp_distance(f["vnorm"], qz.val_a[:, h])        # plain norm: independent of the codes
            assert np.all(u <= NORM_ULP), u.max()
            report["max_vnorm_ulp"] = max(report.get("max_vnorm_ulp", 0), int(u.max()) if u.size else 0)


def rel_err(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)


def check_vec(test: str, workload: str, kind: str, got, ref, ctx=None) -> float:
    """One (sequence, q head) vector of logits or outputs against the oracle: the
    L2 relative error and the largest elementwise error (relative to the largest
    reference magnitude) both within 1e-4; both are recorded for the report."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    l2, el = rel_err(got, ref), elem_err(got, ref)
    report(test, workload, **{f"worst_{kind}_l2": l2, f"worst_{kind}_elem": el, f"{kind}_vectors": 1})
    assert l2 <= REL_TOL and el <= REL_TOL, (ctx, kind, l2, el)
    return max(l2, el)


def build_oracle_cache(w, seq_lens, seed, spare_blocks=0):
    """Quantize a batch of synthetic sequences with the oracle into its own paged cache."""
    cfg = oracle_config(w)
    lay = synth.paged_layout(len(seq_lens), seq_lens, seed, spare_blocks)
    total = int(np.sum(seq_lens))
    k = synth.kv_tensor(w, total, "k", seed)
    v = synth.kv_tensor(w, total, "v", seed)
    cache = O.new_cache(cfg, lay.num_blocks)
    slots = np.concatenate([lay.slots(b, 0, int(n)) for b, n in enumerate(seq_lens)]) if total else np.zeros(0, np.int64)
    if total:
        qz = oracle_quantize(w, k, v)
        O.write_tokens(cfg, cache, slots, qz)
    return lay, cache, k, v, slots


def oracle_decode(w, q, cache, lay, heads=None):
    kcb, vcb = oracle_codebooks(w)
    S = qjl_S(w)
    return O.decode_attention(oracle_config(w), as_f64(q, w), cache, lay.block_tables, lay.seq_lens,
                              1.0 / math.sqrt(w.head_dim), signs(w), kcb, vcb,
                              None if S is None else S.astype(np.float64), heads=heads)
