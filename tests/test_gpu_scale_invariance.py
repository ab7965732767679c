"""Scale invariance of the quantize-append (a metamorphic check at extreme magnitudes).

Multiplying a key by 2^e multiplies its rotation and its norm by 2^e exactly and
leaves the unit vector, hence every code and sign, unchanged; multiplying a value
vector by 2^e scales its min, max and scale exactly and leaves its codes
unchanged (issoh.co.jp "TurboQuantとは？…", 第1段: the norm is kept apart from the
direction; 第2段: per-vector min and scale).  So the pages written for k * 2^e,
v * 2^e must hold the same code bytes as for k, v, and their fp32 scalars must be
exactly 2^e times as large, for e = +40 and -40 (far outside the unit range of
the workloads, inside bf16's range), on the tuned kernels and the generic path.
FP8 keys are left out: E4M3 has a fixed exponent range and saturates, so its
codes are not meant to be scale invariant.
"""
import dataclasses

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "gqa_decode": synth.WORKLOADS["gqa_decode"],
    "qjl": synth.WORKLOADS["qjl"],
    "turbo8v3": synth.WORKLOADS["turbo8v3"],
    "toy": synth.WORKLOADS["toy"],
    "generic d256 qjl": dataclasses.replace(synth.WORKLOADS["qjl"], head_dim=256),
    "generic d64 k4nc": dataclasses.replace(synth.WORKLOADS["gqa_decode"], head_dim=64),
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _scaled(x, w, e):
    """x * 2^e exactly (bf16 bit patterns or fp32)."""
    if w.dtype == "bf16":
        return synth.f32_to_bf16_bits(np.ldexp(synth.bf16_bits_to_f32(x), e).astype(np.float32))
    return np.ldexp(np.asarray(x, np.float32), e).astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("e", [40, -40])
def test_append_is_scale_invariant(name, e):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = CASES[name]
    print(f"[scale invariance] {name} 2^{e}", flush=True)
    n = 200
    k = synth.kv_tensor(w, n, "k", 61)
    v = synth.kv_tensor(w, n, "v", 61)
    slots = np.random.default_rng(62).permutation(16 * 16)[:n].astype(np.int64)
    ctx = H.make_context(w)
    cfg = H.oracle_config(w)
    pages = []
    for kk, vv in ((k, v), (_scaled(k, w, e), _scaled(v, w, e))):
        cache = PagedKVCache(ctx, 16, fill=0xA5)
        cache.append(H.upload(kk, w, torch), H.upload(vv, w, torch), torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        pages.append(cache.data.cpu().numpy())
    for h in range(w.num_kv_heads):
        a = H.O.read_tokens(cfg, pages[0], slots, h)
        b = H.O.read_tokens(cfg, pages[1], slots, h)
        for name_f in a:
            if name_f in ("kcodes", "vcodes", "ksigns"):
                assert np.array_equal(a[name_f], b[name_f]), (name_f, h)
            else:   # fp32 scalars: norms, residual norms, value min / scale or norm
                assert np.array_equal(np.ldexp(a[name_f], e), b[name_f]), (name_f, h)
