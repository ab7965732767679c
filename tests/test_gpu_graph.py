"""GPU tests of HIP graph capture of the hot-path calls (a serving loop replays its
decode step as a graph; the bench times the steps that way).

One graph holds a decode step (the one-launch append-decode, or for PolarQuant
keys also append then decode), a plain decode, a dequantize_rows call and a
whole-batch append into a second cache.  It is
replayed three times, with eager work (fills of the outputs, an eager decode on
another cache) and synchronizations between the replays, and every replay is
checked against the same calls made eagerly: cache bytes and reconstructed rows
bit-exact, attention outputs within 1e-5 relative per (sequence, q head) vector
(the decode's waves take tiles in arrival order, so the fp32 sums may round
differently from launch to launch).
"""
import dataclasses
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRAPH_TOL = 1e-5
# configurations beyond the named workloads: the generic path (head_dim 256) and the
# tuned decode's head groups (8 and 3 query heads per KV head)
GENERIC = {
    "gqa_decode@d256": dataclasses.replace(synth.WORKLOADS["gqa_decode"], head_dim=256),
    "qjl@group8": dataclasses.replace(synth.WORKLOADS["qjl"], num_kv_heads=2, num_q_heads=16),
    "qjl@group3": dataclasses.replace(synth.WORKLOADS["qjl"], num_kv_heads=2, num_q_heads=6),
}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("name,fused", [("gqa_decode", True), ("qjl", True), ("turbo8v3", True), ("polar3", True),
                                        ("polar3", False), ("gqa_decode@d256", True), ("qjl@group8", True)])
def test_graph_replays_match_eager(name, fused):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = GENERIC.get(name) or synth.WORKLOADS[name]
    print(f"[graph] {name} ({'one launch' if fused else 'append, then decode'})", flush=True)
    lens = np.array([300, 97, 16, 1], np.int64)
    B, T = len(lens), int(lens.max())
    lay = synth.paged_layout(B, lens, 71)
    n = int(lens.sum())
    k = synth.kv_tensor(w, n, "k", 71)
    v = synth.kv_tensor(w, n, "v", 71)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    ctx_rows = np.concatenate([start[b] + np.arange(lens[b] - 1) for b in range(B)]).astype(np.int64)
    ctx_slots = np.concatenate([lay.slots(b, 0, int(lens[b]) - 1) for b in range(B)]).astype(np.int64)
    new_rows = (start + lens - 1).astype(np.int64)
    new_slots = np.array([lay.slots(b, int(lens[b]) - 1, int(lens[b]))[0] for b in range(B)], np.int64)
    all_slots = np.concatenate([lay.slots(b, 0, int(lens[b])) for b in range(B)]).astype(np.int64)
    all_rows = np.concatenate([start[b] + np.arange(lens[b]) for b in range(B)]).astype(np.int64)

    ctx = H.make_context(w)
    dev = lambda a: torch.from_numpy(a).cuda()
    k_ctx, v_ctx = H.upload(k[ctx_rows], w, torch), H.upload(v[ctx_rows], w, torch)
    k_new, v_new = H.upload(k[new_rows], w, torch), H.upload(v[new_rows], w, torch)
    k_all, v_all = H.upload(k[all_rows], w, torch), H.upload(v[all_rows], w, torch)
    q = H.upload(synth.query_tensor(w, B, 71), w, torch)
    tables, seq_lens = dev(lay.block_tables), dev(lay.seq_lens)
    s_ctx, s_new, s_all = dev(ctx_slots), dev(new_slots), dev(all_slots)
    scale = 1.0 / math.sqrt(w.head_dim)
    hkv, d = w.num_kv_heads, w.head_dim

    def make():
        c = PagedKVCache(ctx, lay.num_blocks, fill=0)
        c.append(k_ctx, v_ctx, s_ctx)
        c2 = PagedKVCache(ctx, lay.num_blocks, fill=0)
        bufs = dict(out=torch.zeros((B, w.num_q_heads, d), device="cuda"),
                    out2=torch.zeros((B, w.num_q_heads, d), device="cuda"),
                    kb=torch.zeros((n, hkv, d), dtype=torch.bfloat16, device="cuda"),
                    vb=torch.zeros((n, hkv, d), dtype=torch.bfloat16, device="cuda"))
        return c, c2, bufs

    def calls(c, c2, o):
        if fused:
            c.append_decode(k_new, v_new, q, tables, seq_lens, T, scale, out=o["out"])
        else:
            c.append(k_new, v_new, s_new)
            c.decode(q, tables, seq_lens, T, scale, out=o["out"])
        c.decode(q, tables, seq_lens, T, scale, out=o["out2"])
        c.dequantize_rows(s_all, None, o["kb"], o["vb"])
        c2.append(k_all, v_all, s_all)

    # eager reference
    ce, ce2, oe = make()
    calls(ce, ce2, oe)
    # warm the second set of objects eagerly (workspace allocated outside the capture)
    cg, cg2, og = make()
    cg.decode(q, tables, seq_lens, T, scale, out=og["out2"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(cg, cg2, og)
    torch.cuda.synchronize()
    ref = {key: t.cpu() for key, t in oe.items()}
    ref_data, ref_data2 = ce.data.cpu(), ce2.data.cpu()
    other = torch.zeros_like(oe["out2"])
    for rep in range(3):
        # eager work between the replays: clear what the graph must rewrite
        for t in og.values():
            t.fill_(float("nan"))
        cg2.data.zero_()
        ce.decode(q, tables, seq_lens, T, scale, out=other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cg.data.cpu(), ref_data), rep
        assert torch.equal(cg2.data.cpu(), ref_data2), rep
        assert torch.equal(og["kb"].cpu(), ref["kb"]) and torch.equal(og["vb"].cpu(), ref["vb"]), rep
        for key in ("out", "out2"):
            got, want = og[key].cpu().double().numpy(), ref[key].double().numpy()
            for b in range(B):
                for h in range(w.num_q_heads):
                    assert H.rel_err(got[b, h], want[b, h]) <= GRAPH_TOL, (rep, key, b, h)
        print(f"  replay {rep}: matches the eager calls", flush=True)
