"""GPU parity of the generic path (head_dim 64 and 256; Lloyd-Max, QJL and FP8
keys) against the fp64 oracle, through the C ABI, and of the tuned kernels at
group sizes beyond the named workloads (head_dim 128, the `d128_*` cases: one
head group of 3; two, three and four head groups of 4; groups of 7 and 6 as 4 + 3
and 4 + 2, the latter with PolarQuant keys).

Same bars as the tuned path: codes and packed bytes bit-exact outside the 1e-6
decision band, fp32 scalars within their rounding tolerance, logits and outputs
within 1e-4 per (sequence, q head) vector over identical cache bytes, the
dequantized rows within 1e-5 of the oracle's reconstruction.
"""
import dataclasses
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _w(base, **kw):
    return dataclasses.replace(synth.WORKLOADS[base], **kw)


# name -> (workload, ragged batch lengths)
CASES = {
    "d64_k4nc_v4": (_w("gqa_decode", head_dim=64), [700, 0, 65]),
    "d256_k4nc_v4": (_w("gqa_decode", head_dim=256), [300, 17]),
    "d64_qjl2_v4": (_w("qjl", head_dim=64), [257, 31]),
    "d256_qjl2_v4": (_w("qjl", head_dim=256), [200, 1]),
    "d256_k3nc_v3": (_w("long_3bit", head_dim=256), [333, 64]),
    "d64_k8nc_v3": (_w("turbo8v3", head_dim=64), [150, 0, 47]),
    "d256_toy_lloyd_values": (_w("toy", head_dim=256), [1000]),
    "d128_group8": (_w("gqa_decode", num_kv_heads=2, num_q_heads=16), [400, 90]),
    "d64_group3_qjl3": (_w("k3qjl_v2", head_dim=64, num_kv_heads=2, num_q_heads=6), [300, 5]),
    "d128_group16_qjl": (_w("qjl", num_kv_heads=1, num_q_heads=16), [260, 0]),
    "d128_group12_k3v4": (_w("k3v4_nc", num_kv_heads=2, num_q_heads=24), [300, 65, 1]),
    "d128_group7_qjl3": (_w("k3qjl_v2", num_kv_heads=4, num_q_heads=28), [333, 64]),
    "d128_group6_polar3": (_w("polar3", num_kv_heads=2, num_q_heads=12), [200, 33]),
    "d64_fp8_v4": (_w("k8v4", head_dim=64), [300, 0, 33]),
    "d256_fp8_group8": (_w("k8v4", head_dim=256, num_kv_heads=2, num_q_heads=16), [200, 64]),
    # groups below four at head_dim 64 / 256: the 4-head register arrays with unused heads
    "d256_group2_k4nc": (_w("gqa_decode", head_dim=256, num_kv_heads=4, num_q_heads=8), [130, 64, 1]),
    "d64_group3_k2v2": (_w("gqa_decode", head_dim=64, num_kv_heads=2, num_q_heads=6, key_bits=2, val_bits=2),
                        [517, 16]),
    "d128_group3_k4nc": (_w("gqa_decode", num_kv_heads=2, num_q_heads=6), [260, 77]),
    # 4-bit codes with groups of 16 and of 5: four and two row blocks of the logits MFMA
    "d64_group16_k4nc": (_w("gqa_decode", head_dim=64, num_kv_heads=1, num_q_heads=16), [190, 64]),
    "d256_group5_k4nc": (_w("gqa_decode", head_dim=256, num_kv_heads=1, num_q_heads=5), [150, 3]),
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("name", list(CASES))
def test_generic_append_matches_oracle(name):
    w, lens = CASES[name]
    print(f"[generic append] {name}", flush=True)
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    ctx = H.make_context(w)
    cfg = H.oracle_config(w)
    lay = synth.paged_layout(len(lens), lens, 13, spare_blocks=2)
    total = int(np.sum(lens))
    k = synth.kv_tensor(w, total, "k", 13)
    v = synth.kv_tensor(w, total, "v", 13)
    slots = np.concatenate([lay.slots(b, 0, n) for b, n in enumerate(lens)])
    cache = PagedKVCache(ctx, lay.num_blocks, fill=0xA5)
    cache.append(H.upload(k, w, torch), H.upload(v, w, torch), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got = cache.data.cpu().numpy()
    report = {}
    H.compare_append(w, got, slots, H.oracle_quantize(w, k, v), report)
    assert np.all(got[~H.written_mask(cfg, got.shape, slots)] == 0xA5), "bytes outside the written rows changed"
    H.report("generic append", name, tokens=total * w.num_kv_heads, **report)
    print(f"  {report}")


def test_generic_append_degenerate_vectors_and_invalid_slots():
    w = _w("gqa_decode", head_dim=64)
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    ctx = H.make_context(w)
    cfg = H.oracle_config(w)
    k = synth.kv_tensor(w, 6, "k", 5)
    v = synth.kv_tensor(w, 6, "v", 5)
    k[1] = 0                                                        # zero key
    v[2] = synth.f32_to_bf16_bits(np.full((8, 64), -2.5, np.float32))   # constant values
    slots = np.array([3, 20, 21, -1, 4 * 16, 47], dtype=np.int64)   # -1 and 64 (= num_blocks * 16) skipped
    cache = PagedKVCache(ctx, 4, fill=0xA5)
    cache.append(H.upload(k, w, torch), H.upload(v, w, torch), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got = cache.data.cpu().numpy()
    keep = np.array([0, 1, 2, 5])
    H.compare_append(w, got, slots[keep], H.oracle_quantize(w, k[keep], v[keep]), {})
    assert np.all(got[~H.written_mask(cfg, got.shape, slots[keep])] == 0xA5)
    f = H.O.read_tokens(cfg, got, slots[[1]], 0)
    assert np.all(f["kcodes"] == 8) and f["knorm"][0] == 0.0
    f = H.O.read_tokens(cfg, got, slots[[2]], 0)
    assert np.all(f["vcodes"] == 0) and f["vscale"][0] == 0.0 and f["vmin"][0] == -2.5


def _decode(w, ctx, cache_np, lay, q, max_seq, noalloc=False):
    from kv_cache_vector_randomized_amd import tq
    B = len(lay.seq_lens)
    cache = torch.from_numpy(cache_np).cuda()
    tables = torch.from_numpy(lay.block_tables).cuda()
    lens = torch.from_numpy(lay.seq_lens).cuda()
    qd = H.upload(q, w, torch)
    out = torch.full((B, w.num_q_heads, w.head_dim), float("nan"), device="cuda")
    logits = torch.full((B, w.num_q_heads, max(max_seq, 1)), float("nan"), device="cuda")
    dt = tq.TQ_BF16 if w.dtype == "bf16" else tq.TQ_F32
    if noalloc:
        ctx.decode_attention_noalloc(qd, dt, cache, lay.num_blocks, tables, tables.shape[1], lens, B, max_seq,
                                     1.0 / math.sqrt(w.head_dim), out, logits)
    else:
        ws = torch.zeros(ctx.workspace_bytes(B, max_seq), dtype=torch.uint8, device="cuda")
        ctx.decode_attention(qd, dt, cache, lay.num_blocks, tables, tables.shape[1], lens, B, max_seq,
                             1.0 / math.sqrt(w.head_dim), out, ws, ws.numel(), logits_out=logits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), logits.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_generic_decode_matches_oracle_on_identical_bytes(name):
    w, lens = CASES[name]
    print(f"[generic decode] {name}", flush=True)
    lay, cache_np, _, _, _ = H.build_oracle_cache(w, lens, 23)
    q = synth.query_tensor(w, len(lens), 23)
    max_seq = int(max(lens))
    out, logits = _decode(w, H.make_context(w), cache_np, lay, q, max_seq)
    ref_logits, ref_out = H.oracle_decode(w, q, cache_np, lay)
    worst = 0.0
    for b, n in enumerate(lens):
        for h in range(w.num_q_heads):
            if n == 0:
                assert np.all(out[b, h] == 0)
                continue
            el = H.check_vec("generic decode", name, "logit", logits[b, h, :n], ref_logits[(b, h)], (b, h))
            eo = H.check_vec("generic decode", name, "out", out[b, h], ref_out[b, h], (b, h))
            worst = max(worst, el, eo)
    print(f"  worst relative error {worst:.3e}")


@pytest.mark.parametrize("name", ["d64_k4nc_v4", "d256_qjl2_v4", "d128_group8", "d128_group12_k3v4",
                                  "d128_group7_qjl3"])
def test_generic_noalloc_equals_workspace_decode(name):
    w, lens = CASES[name]
    print(f"[generic no-allocation decode] {name}", flush=True)
    lay, cache_np, _, _, _ = H.build_oracle_cache(w, lens, 29)
    q = synth.query_tensor(w, len(lens), 29)
    ctx = H.make_context(w)
    max_seq = int(max(lens))
    a, la = _decode(w, ctx, cache_np, lay, q, max_seq)
    b, lb = _decode(w, ctx, cache_np, lay, q, max_seq, noalloc=True)
    assert np.array_equal(a, b)
    for i, n in enumerate(lens):
        assert np.array_equal(la[i, :, :n], lb[i, :, :n])


@pytest.mark.parametrize("name", ["d64_k4nc_v4", "d256_qjl2_v4", "d256_toy_lloyd_values", "d128_group8",
                                  "d128_group12_k3v4", "d128_group7_qjl3", "d128_group3_k4nc",
                                  "d256_fp8_group8"])
def test_generic_one_launch_step_matches_oracle(name):
    """tq_append_decode: the new token of every sequence is stored (bytes as the
    oracle's, outside the band), then attended with the context."""
    from kv_cache_vector_randomized_amd import tq
    w, lens = CASES[name]
    print(f"[generic one-launch step] {name}", flush=True)
    lens = [n for n in lens if n > 0]
    B = len(lens)
    full = np.asarray(lens, np.int64)
    ctx_lens = full - 1
    lay = synth.paged_layout(B, full, 31)
    cfg = H.oracle_config(w)
    total = int(full.sum())
    k = synth.kv_tensor(w, total, "k", 31)
    v = synth.kv_tensor(w, total, "v", 31)
    start = np.concatenate([[0], np.cumsum(full)[:-1]])
    ctx_rows = np.concatenate([start[b] + np.arange(int(ctx_lens[b])) for b in range(B)]).astype(np.int64)
    ctx_slots = np.concatenate([lay.slots(b, 0, int(ctx_lens[b])) for b in range(B)])
    new_rows = start + full - 1
    new_slots = np.array([lay.slots(b, int(full[b]) - 1, int(full[b]))[0] for b in range(B)])
    cache_np = H.O.new_cache(cfg, lay.num_blocks)
    if ctx_rows.size:
        H.O.write_tokens(cfg, cache_np, ctx_slots, H.oracle_quantize(w, k[ctx_rows], v[ctx_rows]))
    ctx = H.make_context(w)
    cache = torch.from_numpy(cache_np).cuda()
    tables = torch.from_numpy(lay.block_tables).cuda()
    seq = torch.from_numpy(lay.seq_lens).cuda()
    q = synth.query_tensor(w, B, 31)
    max_seq = int(full.max())
    out = torch.full((B, w.num_q_heads, w.head_dim), float("nan"), device="cuda")
    ws = torch.zeros(ctx.workspace_bytes(B, max_seq), dtype=torch.uint8, device="cuda")
    dt = tq.TQ_BF16 if w.dtype == "bf16" else tq.TQ_F32
    ctx.append_decode(H.upload(k[new_rows], w, torch), H.upload(v[new_rows], w, torch), H.upload(q, w, torch), dt,
                      cache, lay.num_blocks, tables, tables.shape[1], seq, B, max_seq, 1.0 / math.sqrt(w.head_dim),
                      out, ws, ws.numel())
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    H.compare_append(w, got, new_slots, H.oracle_quantize(w, k[new_rows], v[new_rows]), {})
    _, ref = H.oracle_decode(w, q, got, lay)
    o = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in range(w.num_q_heads):
            H.check_vec("generic one-launch step", name, "out", o[b, h], ref[b, h], (b, h))


@pytest.mark.parametrize("name", ["d64_k4nc_v4", "d256_qjl2_v4", "d256_toy_lloyd_values", "d64_k8nc_v3", "d64_fp8_v4"])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_generic_dequantize_matches_oracle(name, bf16_out):
    from kv_cache_vector_randomized_amd import tq
    w, lens = CASES[name]
    print(f"[generic dequantize] {name} bf16={bf16_out}", flush=True)
    lay, cache_np, _, _, slots = H.build_oracle_cache(w, lens, 37)
    ctx = H.make_context(w)
    rng = np.random.default_rng(3)
    pick = np.concatenate([rng.choice(slots, size=min(64, slots.size), replace=False), [-1, lay.num_blocks * 16]])
    n = pick.size
    rows = np.arange(n)[::-1].copy()                     # reversed rows: row n-1-i takes entry i
    odt = torch.bfloat16 if bf16_out else torch.float32
    kb = torch.full((n, w.num_kv_heads, w.head_dim), 7.0, dtype=odt, device="cuda")
    vb = torch.full((n, w.num_kv_heads, w.head_dim), 7.0, dtype=odt, device="cuda")
    ctx.dequantize_rows(torch.from_numpy(cache_np).cuda(), lay.num_blocks, torch.from_numpy(pick).cuda(), n,
                        torch.from_numpy(rows).cuda(), kb, vb, n, tq.TQ_BF16 if bf16_out else tq.TQ_F32)
    torch.cuda.synchronize()
    kg = kb.float().cpu().numpy().astype(np.float64)[rows]
    vg = vb.float().cpu().numpy().astype(np.float64)[rows]
    kcb, vcb = H.oracle_codebooks(w)
    valid = (pick >= 0) & (pick < lay.num_blocks * 16)
    tol = 2.0 ** -8 if bf16_out else 1e-5
    for h in range(w.num_kv_heads):
        rk, rv, _ = H.O.dequantize_slots(H.oracle_config(w), cache_np, pick[valid], h, H.signs(w), kcb, vcb)
        for got, ref in ((kg[valid, h], rk), (vg[valid, h], rv)):
            scale = np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1e-30)
            assert np.all(np.abs(got - ref) <= tol * scale), np.max(np.abs(got - ref) / scale)
        assert np.all(kg[~valid, h] == 0) and np.all(vg[~valid, h] == 0)
