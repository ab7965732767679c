"""The decode entry point that allocates nothing (tq_decode_attention_noalloc, for
callers that cannot allocate device memory or pass a workspace),
called through the C ABI, against tq_decode_attention on the same inputs: two
calls in a row, the second with a smaller batch and shorter contexts, each to
the 1e-4 relative bar per (sequence, q head) vector for outputs and logits (the
two launches may sum in different orders), the first also against the oracle.
A request larger than the static scratch is refused before any launch; on the
generic path the entry point plans fewer splits instead, to fit its scratch."""
import math

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import synth, tq
from tests import gpu_helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _both(ctx, w, cache, lay, q, batch, max_seq):
    """Outputs and logits of both entry points for the first `batch` sequences."""
    tables = torch.from_numpy(np.ascontiguousarray(lay.block_tables[:batch])).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(lay.seq_lens[:batch])).cuda()
    qd = H.upload(np.ascontiguousarray(q[:batch]), w, torch)
    res = []
    for noalloc in (False, True):
        out = torch.full((batch, w.num_q_heads, w.head_dim), float("nan"), device="cuda")
        logits = torch.full((batch, w.num_q_heads, max_seq), float("nan"), device="cuda")
        args = (qd, tq.TQ_BF16, cache, lay.num_blocks, tables, tables.shape[1], lens, batch, max_seq,
                1.0 / math.sqrt(w.head_dim), out)
        if noalloc:
            ctx.decode_attention_noalloc(*args, logits_out=logits)
        else:
            need = ctx.workspace_bytes(batch, max_seq)
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
            ctx.decode_attention(*args, ws, need, logits_out=logits)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().astype(np.float64), logits.cpu().numpy().astype(np.float64)))
    return res


def test_noalloc_decode_matches_workspace_decode_twice():
    w = synth.WORKLOADS["gqa_decode"]
    lens = [3000, 17, 0, 129, 2049, 64, 1, 700]
    print("[noalloc] gqa_decode batch 8 then batch 3", flush=True)
    lay, cache_np, _, _, _ = H.build_oracle_cache(w, lens, 61)
    q = synth.query_tensor(w, len(lens), 61)
    ctx = H.make_context(w)
    cache = torch.from_numpy(cache_np).cuda()
    ref_logits, ref_out = H.oracle_decode(w, q, cache_np, lay)
    for batch, max_seq in ((8, 3000), (3, 200)):
        (o_ws, l_ws), (o_na, l_na) = _both(ctx, w, cache, lay, q, batch, max_seq)
        worst = 0.0
        for b in range(batch):
            n = min(int(lens[b]), max_seq)
            for h in range(w.num_q_heads):
                if n == 0:
                    assert np.all(o_na[b, h] == 0) and np.all(o_ws[b, h] == 0)
                    continue
                e = max(H.rel_err(o_na[b, h], o_ws[b, h]), H.rel_err(l_na[b, h, :n], l_ws[b, h, :n]))
                worst = max(worst, e)
                assert e <= H.REL_TOL, (batch, b, h, e)
                if max_seq >= int(lens[b]):          # the full context: the oracle's result too
                    assert H.rel_err(o_na[b, h], ref_out[b, h]) <= H.REL_TOL
                    assert H.rel_err(l_na[b, h, :n], ref_logits[(b, h)]) <= H.REL_TOL
        print(f"  batch {batch}, max_seq {max_seq}: worst difference between the entry points {worst:.2e}")


def test_noalloc_refuses_more_than_its_scratch_before_launch():
    w = synth.WORKLOADS["gqa_decode"]
    ctx = H.make_context(w)
    batch, max_seq = 2048, 262144                   # 16384 (sequence, kv head) pairs, 64 splits each
    assert ctx.workspace_bytes(batch, max_seq) > tq.STATIC_SCRATCH_BYTES
    small = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = torch.zeros(16, dtype=torch.float32, device="cuda")
    cache = torch.zeros(16 * 8 * 2240, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError) as e:
        ctx.decode_attention_noalloc(small, tq.TQ_BF16, cache, 16, small, 1, small, batch, max_seq, 0.1, out)
    assert e.value.status == tq.TQ_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()


def test_generic_noalloc_plans_fewer_splits_to_fit_its_scratch():
    """head_dim 256, 128 sequences x 1088 tokens x 8 KV heads of 4 query heads: the
    workspace plan (2 splits of 4.2 MB of partials each) exceeds the static scratch,
    so the entry point that allocates nothing plans one split; its outputs and
    logits match the workspace call to the 1e-4 bar (the sums run in another order)."""
    import dataclasses
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = dataclasses.replace(synth.WORKLOADS["gqa_decode"], head_dim=256, batch=128, context=1088)
    B, T = w.batch, w.context
    print("[noalloc] generic head_dim 256, 128 x 1088 tokens", flush=True)
    ctx = H.make_context(w)
    assert ctx.workspace_bytes(B, T) > tq.STATIC_SCRATCH_BYTES
    lay = synth.paged_layout(B, [T] * B, 71)
    gen = torch.Generator(device="cuda").manual_seed(71)
    k = torch.randn((B * T, w.num_kv_heads, w.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((B * T, w.num_kv_heads, w.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    slots = torch.from_numpy(np.concatenate([lay.slots(b, 0, T) for b in range(B)])).cuda()
    cache = PagedKVCache(ctx, lay.num_blocks)
    cache.append(k, v, slots)
    torch.cuda.synchronize()
    del k, v
    q = synth.query_tensor(w, B, 71)
    (o_ws, l_ws), (o_na, l_na) = _both(ctx, w, cache.data, lay, q, B, T)
    worst = 0.0
    for b in range(B):
        for h in range(w.num_q_heads):
            e = max(H.rel_err(o_na[b, h], o_ws[b, h]), H.rel_err(l_na[b, h], l_ws[b, h]))
            worst = max(worst, e)
            assert e <= H.REL_TOL, (b, h, e)
    print(f"  worst difference between the entry points {worst:.2e}")
