"""Pins for the oracle's QJL estimator and decode attention (CPU only)."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as O
from kv_cache_vector_randomized_amd import synth


def _qjl_estimates(q, k, signs, cb, n_draws, seed):
    rng = np.random.default_rng(seed)
    ests = []
    for _ in range(n_draws):
        S = rng.standard_normal((128, 128))
        kq = O.quantize_keys(k[None], signs, cb, "lloyd_qjl", S)
        fields = {"ksigns": kq.qjl_bits, "kres": kq.qjl_norm}
        stage1 = O.dequantize_keys(kq.codes, kq.norm, signs, cb)[0] @ q
        ests.append((stage1, O.qjl_correction(q, signs, S, fields)[0]))
    return np.array(ests), kq


def test_qjl_is_unbiased_and_variance_matches_closed_form():
    """lilting.ch QJL section: the corrected score is an unbiased estimate of <q, k>.
    For g ~ N(0, I): E[(g.a) sign(g.b)] = sqrt(2/pi) a.b/||b||; the variance of the
    m-row estimate of <q, r> is ((pi/2)||q||^2||r||^2 - (q.r)^2)/m."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128) * 2
    signs = synth.sign_vector(5)
    cb = O.codebook(2, 128)
    est, kq = _qjl_estimates(q, k, signs, cb, 2000, 12)
    stage1 = est[0, 0]
    r = k - O.dequantize_keys(kq.codes, kq.norm, signs, cb)[0]
    truth_corr = r @ q
    corr = est[:, 1]
    se = corr.std(ddof=1) / math.sqrt(len(corr))
    assert abs(corr.mean() - truth_corr) < 4 * se
    assert abs((stage1 + corr.mean()) - k @ q) < 4 * se
    var_theory = ((math.pi / 2) * (q @ q) * (r @ r) - (q @ r) ** 2) / 128
    ratio = corr.var(ddof=1) / var_theory
    assert 0.85 < ratio < 1.15, ratio


def test_mse_quantizer_biases_inner_products():
    """issoh.co.jp stage-2 section: the MSE-optimal stage-1 quantizer shrinks inner products
    (on average by 1 - distortion for unit vectors); the QJL stage removes the shrink."""
    d, n = 128, 4000
    rng = np.random.default_rng(21)
    signs = synth.sign_vector(5)
    cb = O.codebook(2, d)
    k = rng.standard_normal((n, d))
    kq = O.quantize_keys(k, signs, cb, "lloyd")
    k_hat = O.dequantize_keys(kq.codes, kq.norm, signs, cb)
    shrink = ((k_hat * k).sum(1) / (k * k).sum(1)).mean()
    mse = ((k / np.linalg.norm(k, axis=1, keepdims=True)
            - k_hat / np.linalg.norm(k, axis=1, keepdims=True)) ** 2).sum(1).mean()
    assert shrink < 0.9
    assert abs(shrink - (1 - mse)) < 0.01


def test_attention_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((7, 16))
    k = np.zeros((7, 16))
    lg, out = O.attention_one(rng.standard_normal(16), k, v, 0.5)
    assert np.allclose(out, v.mean(0)) and np.allclose(lg, 0)            # equal logits -> mean
    lg, out = O.attention_one(rng.standard_normal(16), k[:1], v[:1], 0.5)
    assert np.allclose(out, v[0])                                        # one token -> that value
    # two tokens, logits 0 and ln 3 -> p = (1/4, 3/4)
    q = np.zeros(16); q[0] = 1.0
    k2 = np.zeros((2, 16)); k2[1, 0] = 2 * math.log(3.0)
    lg, out = O.attention_one(q, k2, v[:2], 0.5)
    assert np.allclose(lg, [0, math.log(3.0)])
    assert np.allclose(out, 0.25 * v[0] + 0.75 * v[1])
    # one dominant logit
    k3 = np.zeros((7, 16)); k3[4, 0] = 1e4
    assert np.allclose(O.attention_one(q, k3, v, 1.0)[1], v[4])
    # empty context
    assert np.all(O.attention_one(q, k[:0], v[:0], 1.0)[1] == 0)


def test_blockwise_softmax_merge_equals_direct():
    """The split-context (log-sum-exp) merge the GPU uses is an exact re-association."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal(1000) * 4
    v = rng.standard_normal((1000, 8))
    p = np.exp(lg - lg.max()); p /= p.sum()
    direct = p @ v
    parts = []
    for s in range(0, 1000, 137):
        m = lg[s:s + 137].max()
        e = np.exp(lg[s:s + 137] - m)
        parts.append((m, e.sum(), e @ v[s:s + 137]))
    M = max(m for m, _, _ in parts)
    num = sum(math.exp(m - M) * o for m, _, o in parts)
    den = sum(math.exp(m - M) * l for m, l, _ in parts)
    assert np.allclose(num / den, direct, rtol=1e-12, atol=1e-14)


def _small_cache(cfg, seq_lens, seed, S=None):
    lay = synth.paged_layout(len(seq_lens), seq_lens, seed)
    rng = np.random.default_rng(seed)
    signs = synth.sign_vector(seed)
    kcb = O.codebook(cfg.key_bits, cfg.head_dim)
    vcb = O.codebook(cfg.val_bits, cfg.head_dim) if cfg.val_mode == "lloyd" else None
    cache = O.new_cache(cfg, lay.num_blocks)
    kv = {}
    for b, n in enumerate(seq_lens):
        k = rng.standard_normal((n, cfg.num_kv_heads, cfg.head_dim))
        v = rng.standard_normal((n, cfg.num_kv_heads, cfg.head_dim))
        O.quantize_append(cfg, cache, k, v, lay.slots(b, 0, n), signs, kcb, vcb, S)
        kv[b] = (k, v)
    return lay, cache, signs, kcb, vcb, kv


def test_gqa_head_mapping_and_paging():
    """q head h reads kv head h // (Hq/Hkv); pages may sit anywhere (block tables)."""
    cfg = O.Config(128, 2, 8, 4, "lloyd_nc", 4, "uniform")
    lay, cache, signs, kcb, vcb, kv = _small_cache(cfg, [37, 16], 4)
    q = np.random.default_rng(9).standard_normal((2, 8, 128))
    lg, out = O.decode_attention(cfg, q, cache, lay.block_tables, lay.seq_lens, 1 / math.sqrt(128),
                                 signs, kcb, vcb)
    for b, n in enumerate([37, 16]):
        for h in range(8):
            kvh = h // 4
            f = O.read_tokens(cfg, cache, lay.slots(b, 0, n), kvh)
            k_hat = O.dequantize_keys(f["kcodes"], f["knorm"], signs, kcb)
            v_hat = O.dequantize_values_uniform(f["vcodes"], f["vmin"], f["vscale"])
            l2, o2 = O.attention_one(q[b, h], k_hat, v_hat, 1 / math.sqrt(128))
            assert np.allclose(lg[(b, h)], l2) and np.allclose(out[b, h], o2)
            # against the unquantized attention the error stays small
            ref_l = kv[b][0][:, kvh] @ q[b, h] / math.sqrt(128)
            assert np.corrcoef(ref_l, l2)[0, 1] > 0.98


def test_decode_with_lloyd_values_and_qjl_runs_and_is_consistent():
    cfg = O.Config(128, 1, 1, 4, "lloyd", 4, "lloyd")
    lay, cache, signs, kcb, vcb, kv = _small_cache(cfg, [40], 6)
    q = np.random.default_rng(3).standard_normal((1, 1, 128))
    lg, out = O.decode_attention(cfg, q, cache, lay.block_tables, lay.seq_lens, 0.1, signs, kcb, vcb)
    k, v = kv[0]
    ref = np.exp(0.1 * k[:, 0] @ q[0, 0]); ref /= ref.sum()
    assert np.linalg.norm(out[0, 0] - ref @ v[:, 0]) / np.linalg.norm(ref @ v[:, 0]) < 0.2
    S = synth.qjl_matrix().astype(np.float64)
    cfg5 = O.Config(128, 2, 8, 2, "lloyd_qjl", 4, "uniform")
    lay, cache, signs, kcb, vcb, kv = _small_cache(cfg5, [33], 7, S)
    q = np.random.default_rng(4).standard_normal((1, 8, 128))
    lg, out = O.decode_attention(cfg5, q, cache, lay.block_tables, lay.seq_lens, 1.0, signs, kcb, S=S)
    f = O.read_tokens(cfg5, cache, lay.slots(0, 0, 33), 0)
    st1 = O.dequantize_keys(f["kcodes"], f["knorm"], signs, kcb) @ q[0, 0]
    assert np.allclose(lg[(0, 0)], st1 + O.qjl_correction(q[0, 0], signs, S, f))
