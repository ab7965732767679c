"""Value sums at the longest context, with a softmax chosen to make the fixed-point
value weights round the same way everywhere.

The decode adds up p_t * scale_t * code_t on the int8 MFMA, the weights p_t * scale_t
of a 64-token tile rounded to a fixed-point grid of 2^-27 times a bound on the
tile's largest weight of each head.  Here one token carries weight 1 and 262143
identical tokens carry 2^-g each (g = 12, 16, 20, 24 for the four query heads:
the tail is 64x, 4x, 1/4 and 1/64 of the first token's weight).  All tail tokens
have the same fields, so all their weights round by the same amount in the same
direction: a grid tied to the largest value scale alone (not to the weights)
would leave the tail's weights with about 27 - g significant bits and an error
that grows with the context: a model of that rounding puts 7e-4 to 2.5e-3 on
the outputs of the heads with g = 16, 20, 24.  With the grid
tied to each tile's largest weight the error bound does not depend on the
length; every head must meet the 1e-4 bar against the oracle over the same bytes.
"""
import dataclasses
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

T = 262144
GAPS = (12, 16, 20, 24)             # log2 of the first token's weight over a tail token's


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _peaked_case():
    w = dataclasses.replace(synth.WORKLOADS["gqa_decode"], num_kv_heads=1, num_q_heads=4, batch=1, context=T)
    cfg = H.oracle_config(w)
    rng = np.random.default_rng(1234)
    to_bf16 = lambda x: synth.f32_to_bf16_bits(np.asarray(x, np.float32))
    k_tail = to_bf16(rng.standard_normal(128))
    k_first = to_bf16(2.0 * synth.bf16_bits_to_f32(k_tail))     # same direction: same codes, twice the norm
    v_tail = to_bf16(rng.standard_normal(128))
    v_first = to_bf16(rng.standard_normal(128))
    k2 = np.stack([k_first, k_tail])[:, None, :]
    v2 = np.stack([v_first, v_tail])[:, None, :]
    qz = H.oracle_quantize(w, k2, v2)
    assert np.array_equal(qz.key.codes[0], qz.key.codes[1])
    assert qz.key.norm[0, 0] == 2.0 * qz.key.norm[1, 0]
    # the tail's logit is scale * q . k_hat_tail and the first token's twice that, so a
    # query along k_hat_tail with logit g ln 2 puts 2^-g on every tail token
    kcb, _ = H.oracle_codebooks(w)
    k_hat = H.O.dequantize_keys(qz.key.codes[1, 0], qz.key.norm[1, 0], H.signs(w), kcb)
    scale = 1.0 / math.sqrt(w.head_dim)
    u = k_hat / np.linalg.norm(k_hat)
    q = np.stack([to_bf16(u * g * math.log(2.0) / (scale * np.linalg.norm(k_hat))) for g in GAPS])[None]
    # pages: the first holds the first token and 15 tail tokens, every other page 16 tail tokens
    lay = synth.paged_layout(1, [T], 77)
    small = H.O.new_cache(cfg, 2, fill=0)
    H.O.write_tokens(cfg, small, np.arange(32), dataclasses.replace(
        qz, key=dataclasses.replace(qz.key, codes=qz.key.codes[[0] + [1] * 31], norm=qz.key.norm[[0] + [1] * 31]),
        val_codes=qz.val_codes[[0] + [1] * 31], val_a=qz.val_a[[0] + [1] * 31], val_b=qz.val_b[[0] + [1] * 31]))
    cache = np.empty((lay.num_blocks,) + small.shape[1:], np.uint8)
    cache[:] = small[1]
    cache[lay.block_tables[0, 0]] = small[0]
    return w, lay, cache, q, scale


def test_peaked_softmax_over_262144_identical_tail_tokens():
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    print("[value precision] 262144 tokens, one dominant token, identical tail", flush=True)
    w, lay, cache_np, q, scale = _peaked_case()
    ref_logits, ref_out = H.oracle_decode(w, q, cache_np, lay)
    for h, g in enumerate(GAPS):                 # the construction gives the intended weights
        lg = ref_logits[(0, h)]
        assert abs((lg[0] - lg[1]) / math.log(2.0) - g) < 0.25 and np.all(lg[1:] == lg[1])
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks)
    cache.data.copy_(torch.from_numpy(cache_np))
    out = cache.decode(H.upload(q, w, torch), torch.from_numpy(lay.block_tables).cuda(),
                       torch.from_numpy(lay.seq_lens).cuda(), T, scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for h, g in enumerate(GAPS):
        e = H.check_vec("value precision, peaked softmax", f"T{T} g{g}", "out", out[0, h], ref_out[0, h], (0, h))
        print(f"  tail weight 2^-{g}: relative error {e:.2e}", flush=True)
        worst = max(worst, e)
    print(f"  worst {worst:.2e}")
