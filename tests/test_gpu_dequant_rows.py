"""GPU tests of incremental dequantization (tq_dequantize_rows): a running buffer
that receives the context once and then only each step's new tokens (the
turboquant-vllm write-up, "Incremental dequantization").

* after a prefill and several one-token steps, the running buffer equals the
  whole cache reconstructed at once (bit-exact: the same arithmetic per token),
  the bf16 buffer is within bf16 rounding (2^-8 relative per element) of it,
  and the reconstruction matches the oracle's over the GPU bytes (1e-5 relative
  per vector);
* rows that were never listed keep their sentinel; rows outside the buffer are
  skipped; slots outside the cache give zero rows;
* attention computed densely over the running buffer equals the fused decode
  over the packed cache (1e-4 relative per (sequence, q head) vector).
"""
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _dense_attention(q, kbuf, vbuf, base, n, group, scale):
    """fp64 softmax attention of one query over rows base..base+n of the buffer."""
    k = kbuf[base:base + n].astype(np.float64)
    v = vbuf[base:base + n].astype(np.float64)
    out = np.zeros((q.shape[0], k.shape[-1]))
    for h in range(q.shape[0]):
        logits = scale * (k[:, h // group] @ q[h])
        p = np.exp(logits - logits.max())
        out[h] = (p / p.sum()) @ v[:, h // group]
    return out


@pytest.mark.parametrize("name", ["toy", "gqa_decode", "long_3bit", "qjl", "k3v4_nc", "k3qjl_v2", "k8v4", "turbo8v3",
                                  "polar3"])
def test_incremental_buffer_equals_full_dequantize(name):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS[name]
    print(f"[dequantize_rows] {name}", flush=True)
    steps = 5
    ctx_lens = np.array([70, 33, 5] if w.num_q_heads > 1 else [70], np.int64)
    B = len(ctx_lens)
    lens = ctx_lens + steps
    tmax = int(lens.max()) + 3                   # spare rows stay untouched
    lay = synth.paged_layout(B, lens, 61)
    k = synth.kv_tensor(w, int(lens.sum()), "k", 61)
    v = synth.kv_tensor(w, int(lens.sum()), "v", 61)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks, fill=0)
    hkv, d = w.num_kv_heads, w.head_dim
    bufs = {dt: (torch.full((B * tmax, hkv, d), float("nan"), dtype=dt, device="cuda"),
                 torch.full((B * tmax, hkv, d), float("nan"), dtype=dt, device="cuda"))
            for dt in (torch.float32, torch.bfloat16)}

    def put(b, p0, p1):
        """Quantize positions p0..p1-1 of every sequence, then dequantize them into the buffers."""
        rows_src = np.concatenate([start[i] + np.arange(p0, p1) for i in b]).astype(np.int64)
        slots = np.concatenate([lay.slots(i, p0, p1) for i in b]).astype(np.int64)
        dst = np.concatenate([i * tmax + np.arange(p0, p1) for i in b]).astype(np.int64)
        cache.append(H.upload(k[rows_src], w, torch), H.upload(v[rows_src], w, torch), torch.from_numpy(slots).cuda())
        for kb, vb in bufs.values():
            cache.dequantize_rows(torch.from_numpy(slots).cuda(), torch.from_numpy(dst).cuda(), kb, vb)

    # prefill: each sequence's context at once, then one token per step
    for b in range(B):
        put([b], 0, int(ctx_lens[b]))
    for s in range(steps):
        for b in range(B):
            put([b], int(ctx_lens[b]) + s, int(ctx_lens[b]) + s + 1)
    torch.cuda.synchronize()

    all_slots = np.concatenate([lay.slots(b, 0, int(lens[b])) for b in range(B)]).astype(np.int64)
    kf, vf = cache.dequantize(torch.from_numpy(all_slots).cuda())
    torch.cuda.synchronize()
    kf, vf = kf.cpu(), vf.cpu()
    k32, v32 = (t.cpu() for t in bufs[torch.float32])
    k16, v16 = (t.cpu() for t in bufs[torch.bfloat16])
    off = 0
    for b in range(B):
        n = int(lens[b])
        r = slice(b * tmax, b * tmax + n)
        assert torch.equal(k32[r], kf[off:off + n]) and torch.equal(v32[r], vf[off:off + n]), b
        for got, ref in ((k16[r], kf[off:off + n]), (v16[r], vf[off:off + n])):
            # bf16 rows: round-to-nearest-even of an fp32 reconstruction whose butterfly
            # order may differ from the fp32 kernel's (a few elements one bf16 ulp apart)
            g = got.double()
            rr = ref.double()
            row = rr.abs().amax(dim=-1, keepdim=True)
            assert ((g - rr).abs() <= 2.0 ** -8 * rr.abs() + 1e-6 * row).all(), b
            same = (got.view(torch.int16) == ref.to(torch.bfloat16).view(torch.int16)).double().mean().item()
            assert same > 0.99, (b, same)
        spare = slice(b * tmax + n, (b + 1) * tmax)
        assert torch.isnan(k32[spare]).all() and torch.isnan(v16[spare]).all(), "an unlisted row changed"
        off += n

    # the reconstruction itself, against the oracle over the GPU bytes
    cache_np = cache.data.cpu().numpy()
    kcb, vcb = H.oracle_codebooks(w)
    kf, vf = kf.numpy(), vf.numpy()
    worst = 0.0
    for h in range(hkv):
        rk, rv, _ = H.O.dequantize_slots(H.oracle_config(w), cache_np, all_slots, h, H.signs(w),
                                         kcb, vcb)
        for i in range(len(all_slots)):
            e = max(H.rel_err(kf[i, h], rk[i]), H.rel_err(vf[i, h], rv[i]))
            worst = max(worst, e)
            assert e <= 1e-5, (h, i, e)
    print(f"  running buffer == full dequantize; worst relative error vs oracle {worst:.2e}", flush=True)

    # dense attention over the running buffer vs the fused decode over the packed cache
    if w.key_mode != "lloyd_qjl":               # the buffer holds stage 1 only; QJL decode adds the residual term
        q = synth.query_tensor(w, B, 61)
        scale = 1.0 / math.sqrt(d)
        out = cache.decode(H.upload(q, w, torch), torch.from_numpy(lay.block_tables).cuda(),
                           torch.from_numpy(lay.seq_lens).cuda(), int(lens.max()), scale)
        torch.cuda.synchronize()
        out = out.cpu().numpy().astype(np.float64)
        qf = H.as_f64(q, w)
        kb, vb = k32.numpy(), v32.numpy()
        group = w.num_q_heads // hkv
        for b in range(B):
            ref = _dense_attention(qf[b], kb, vb, b * tmax, int(lens[b]), group, scale)
            for h in range(w.num_q_heads):
                assert H.rel_err(out[b, h], ref[h]) <= H.REL_TOL, (b, h)
        print("  dense attention over the running buffer == fused decode", flush=True)


def test_rows_outside_buffer_and_slots_outside_cache():
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS["gqa_decode"]
    lens = [40]
    lay, cache_np, k, v, slots = H.build_oracle_cache(w, lens, 63)
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks)
    cache.data.copy_(torch.from_numpy(cache_np))
    hkv, d = w.num_kv_heads, w.head_dim
    nrows = 8
    ask = np.array([slots[3], slots[7], -1, lay.num_blocks * 16, slots[9], slots[11]], np.int64)
    rows = np.array([0, 5, 2, 3, -1, nrows], np.int64)          # the last two rows are outside the buffer
    kb = torch.full((nrows, hkv, d), float("nan"), device="cuda")
    vb = torch.full((nrows, hkv, d), float("nan"), device="cuda")
    cache.dequantize_rows(torch.from_numpy(ask).cuda(), torch.from_numpy(rows).cuda(), kb, vb)
    kf, vf = cache.dequantize(torch.from_numpy(ask).cuda())
    torch.cuda.synchronize()
    kb, vb, kf, vf = kb.cpu(), vb.cpu(), kf.cpu(), vf.cpu()
    for i, r in enumerate(rows[:4]):
        assert torch.equal(kb[r], kf[i]) and torch.equal(vb[r], vf[i])
    assert (kb[2] == 0).all() and (vb[3] == 0).all(), "a slot outside the cache must give a zero row"
    for r in (1, 4, 6, 7):
        assert torch.isnan(kb[r]).all() and torch.isnan(vb[r]).all(), r
    # rows = None: row i, the same as tq_dequantize
    k2 = torch.empty((len(ask), hkv, d), device="cuda")
    v2 = torch.empty_like(k2)
    cache.dequantize_rows(torch.from_numpy(ask).cuda(), None, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(k2.cpu(), kf) and torch.equal(v2.cpu(), vf)
