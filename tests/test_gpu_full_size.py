"""GPU parity at the full sizes the benchmark runs (the five configurations and the
serving presets), in the launch configuration it times (same shapes, same split
plan, no logits buffer), checked on samples the oracle computes one by one:

* append: every field of 512 seeded random tokens (all KV heads) against the
  oracle's quantization of those tokens, to the same bars as the small cases;
* decode: outputs of whole (sequence, KV head) groups of query heads against the
  oracle attending over the GPU-written cache bytes of that sequence (1e-4
  relative per vector); a second launch with a logits buffer checks the logits
  of the same heads and its outputs must meet the same bar.  Tiles are handed to
  waves dynamically, so the fp32 summation order differs between launches (the
  outputs cancel, so that shows at about 1e-5); on every head the two launches
  must agree within the oracle bar;
* the one-launch step (tq_append_decode), the benchmark's default launch: the
  cache holds positions 0..T-2 of every sequence, one launch quantizes position
  T-1 and attends over all T; the new tokens' fields against the oracle's
  quantization, sampled groups against the oracle over the GPU-written bytes.
"""
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# workload -> (sequence, kv head) pairs whose query heads are checked
SAMPLES = {
    "gqa_decode": [(0, 0), (7, 3), (15, 7)],
    "long_3bit": [(0, 2), (3, 6)],
    "prefill_append": [(0, 0), (0, 5)],
    "qjl": [(1, 1), (6, 4)],
    # the serving presets at the shapes the benchmark runs them
    "k3v4_nc": [(2, 1), (13, 6)],
    "k3qjl_v2": [(0, 3), (7, 5)],
    "k8v4": [(4, 0), (11, 7)],
    "turbo8v3": [(1, 2), (14, 4)],
    "polar3": [(3, 3), (9, 6)],
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_append_and_decode_sampled(name):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS[name]
    print(f"[full size] {name}", flush=True)
    B, T, G = w.batch, w.context, w.num_q_heads // w.num_kv_heads
    lay = synth.paged_layout(B, [T] * B, w.seed)          # the benchmark's layout and inputs
    k = synth.kv_tensor(w, B * T, "k")
    v = synth.kv_tensor(w, B * T, "v")
    q = synth.query_tensor(w)
    slots = np.concatenate([lay.slots(b, 0, T) for b in range(B)])
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks)
    cache.append(H.upload(k, w, torch), H.upload(v, w, torch), torch.from_numpy(slots).cuda())
    tables = torch.from_numpy(lay.block_tables).cuda()
    lens = torch.from_numpy(lay.seq_lens).cuda()
    qd = H.upload(q, w, torch)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = cache.decode(qd, tables, lens, T, scale).cpu().numpy().astype(np.float64)
    logits = torch.full((B, w.num_q_heads, T), float("nan"), device="cuda")
    out2 = cache.decode(qd, tables, lens, T, scale, logits=logits).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    drift = max(H.rel_err(out2[b, h], out[b, h]) for b in range(B) for h in range(w.num_q_heads))
    assert drift <= H.REL_TOL, f"two launches differ by {drift:.2e}"
    logits = logits.cpu().numpy().astype(np.float64)
    cache_np = cache.data.cpu().numpy()

    # append: sampled tokens, every KV head
    pick = np.sort(np.random.default_rng(99).choice(B * T, size=512, replace=False))
    qz = H.oracle_quantize(w, k[pick], v[pick])
    report = {}
    H.compare_append(w, cache_np, slots[pick], qz, report)
    H.report("full size append (512 tokens)", name, tokens=512 * w.num_kv_heads, **report)
    print(f"  append sample: {report}")

    # decode: whole kv-head groups of query heads of sampled sequences
    heads = [(b, kvh * G + i) for b, kvh in SAMPLES[name] for i in range(G)]
    ref_logits, ref_out = H.oracle_decode(w, q, cache_np, lay, heads=heads)
    worst = 0.0
    for b, h in heads:
        el = H.check_vec("full size decode", name, "logit", logits[b, h], ref_logits[(b, h)], (b, h))
        eo = H.check_vec("full size decode", name, "out", out[b, h], ref_out[b, h], (b, h))
        eo2 = H.check_vec("full size decode", name, "out", out2[b, h], ref_out[b, h], (b, h))
        worst = max(worst, el, eo, eo2)
    print(f"  decode sample of {len(heads)} heads: worst relative error {worst:.3e}; launches differ by {drift:.2e}")


@pytest.mark.parametrize("name", [n for n in SAMPLES if n != "prefill_append"])
def test_full_size_one_launch_step_sampled(name):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS[name]
    print(f"[full size, one launch] {name}", flush=True)
    B, T, G = w.batch, w.context, w.num_q_heads // w.num_kv_heads
    lay = synth.paged_layout(B, [T] * B, w.seed)
    k = synth.kv_tensor(w, B * T, "k")
    v = synth.kv_tensor(w, B * T, "v")
    q = synth.query_tensor(w)
    ctx_rows = np.concatenate([b * T + np.arange(T - 1) for b in range(B)])
    ctx_slots = np.concatenate([lay.slots(b, 0, T - 1) for b in range(B)])
    new_rows = np.arange(B) * T + T - 1
    new_slots = np.array([lay.slots(b, T - 1, T)[0] for b in range(B)], np.int64)
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks)
    cache.append(H.upload(k[ctx_rows], w, torch), H.upload(v[ctx_rows], w, torch), torch.from_numpy(ctx_slots).cuda())
    out = cache.append_decode(H.upload(k[new_rows], w, torch), H.upload(v[new_rows], w, torch), H.upload(q, w, torch),
                              torch.from_numpy(lay.block_tables).cuda(), torch.from_numpy(lay.seq_lens).cuda(), T,
                              1.0 / math.sqrt(w.head_dim))
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    cache_np = cache.data.cpu().numpy()
    report = {}
    H.compare_append(w, cache_np, new_slots, H.oracle_quantize(w, k[new_rows], v[new_rows]), report)
    H.report("full size one-launch step (new tokens)", name, tokens=len(new_slots) * w.num_kv_heads, **report)
    print(f"  new tokens: {report}")
    heads = [(b, kvh * G + i) for b, kvh in SAMPLES[name] for i in range(G)]
    _, ref_out = H.oracle_decode(w, q, cache_np, lay, heads=heads)
    worst = 0.0
    for b, h in heads:
        worst = max(worst, H.check_vec("full size one-launch step", name, "out", out[b, h], ref_out[b, h], (b, h)))
    print(f"  one-launch step, {len(heads)} sampled heads: worst relative error {worst:.3e}")
