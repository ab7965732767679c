"""GPU tests at the limits of one decode call.

* 16384 (sequence, KV head) pairs, the most one call takes (batch 2048 x 8 KV
  heads, ragged lengths 0..40): the one-launch step, then the plain decode over
  the resulting cache, against the oracle attending over the GPU-written bytes
  for 48 sampled sequences (every query head; 1e-4 relative per vector);
  sequences of length 0 give zero rows.  One sequence more (16392 pairs) is
  refused with TQ_ERR_UNSUPPORTED before any launch.
* One sequence of 262144 tokens on one KV head with 4 query heads: 4096 tiles
  split 256 ways, so the last work-group to finish merges 256 partials; the
  one-launch step and the plain decode against the oracle on all four heads.
"""
import dataclasses
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


def _step_and_check(w, lens, seed, sample):
    """Cache of positions 0..len-2 of every sequence, then one append-decode launch
    with position len-1 and one plain decode; both against the oracle on the
    sampled sequences (all query heads), zero rows for empty sequences."""
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    lens = np.asarray(lens, np.int64)
    B, T = len(lens), int(lens.max())
    lay = synth.paged_layout(B, lens, seed)
    n = int(lens.sum())
    k = synth.kv_tensor(w, n, "k", seed)
    v = synth.kv_tensor(w, n, "v", seed)
    q = synth.query_tensor(w, B, seed)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    ctx_rows = np.concatenate([start[b] + np.arange(max(int(lens[b]) - 1, 0)) for b in range(B)]).astype(np.int64)
    ctx_slots = np.concatenate([lay.slots(b, 0, max(int(lens[b]) - 1, 0)) for b in range(B)]).astype(np.int64)
    has_new = lens > 0
    new_rows = np.where(has_new, start + lens - 1, 0)
    k_new, v_new = k[new_rows].copy(), v[new_rows].copy()
    k_new[~has_new] = 0
    v_new[~has_new] = 0
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks, fill=0)
    if len(ctx_rows):
        cache.append(H.upload(k[ctx_rows], w, torch), H.upload(v[ctx_rows], w, torch),
                     torch.from_numpy(ctx_slots).cuda())
    tables = torch.from_numpy(lay.block_tables).cuda()
    seq = torch.from_numpy(lay.seq_lens).cuda()
    qd = H.upload(q, w, torch)
    scale = 1.0 / math.sqrt(w.head_dim)
    out1 = cache.append_decode(H.upload(k_new, w, torch), H.upload(v_new, w, torch), qd, tables, seq, T, scale)
    out2 = cache.decode(qd, tables, seq, T, scale)
    torch.cuda.synchronize()
    out1 = out1.cpu().numpy().astype(np.float64)
    out2 = out2.cpu().numpy().astype(np.float64)
    cache_np = cache.data.cpu().numpy()
    assert np.all(out1[~has_new] == 0) and np.all(out2[~has_new] == 0)
    heads = [(int(b), h) for b in sample for h in range(w.num_q_heads)]
    _, ref = H.oracle_decode(w, q, cache_np, lay, heads=heads)
    worst = 0.0
    tag = f"limits B{B} T{T}"
    for b, h in heads:
        e1 = H.check_vec(tag + " one-launch step", w.name, "out", out1[b, h], ref[b, h], (b, h))
        e2 = H.check_vec(tag + " decode", w.name, "out", out2[b, h], ref[b, h], (b, h))
        worst = max(worst, e1, e2)
    return worst


def test_most_pairs_one_call_takes():
    w = dataclasses.replace(synth.WORKLOADS["gqa_decode"], batch=2048, context=40)
    print("[limits] 2048 sequences x 8 kv heads", flush=True)
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 41, size=2048)
    lens[:3] = [0, 1, 40]
    sample = np.concatenate([[1, 2], rng.choice(np.nonzero(lens > 0)[0], size=46, replace=False)])
    worst = _step_and_check(w, lens, 91, np.unique(sample))
    print(f"  worst relative error {worst:.2e}", flush=True)


def test_one_sequence_more_is_refused():
    from kv_cache_vector_randomized_amd import tq
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = dataclasses.replace(synth.WORKLOADS["gqa_decode"], batch=2049, context=1)
    lay = synth.paged_layout(2049, np.ones(2049, np.int64), 92)
    cache = PagedKVCache(H.make_context(w), lay.num_blocks, fill=0)
    q = torch.zeros((2049, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((2049, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    tables = torch.from_numpy(lay.block_tables).cuda()
    seq = torch.from_numpy(lay.seq_lens).cuda()
    with pytest.raises(tq.TQError) as e:
        cache.decode(q, tables, seq, 1, 1.0)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TQError):
        cache.append_decode(kn, kn, q, tables, seq, 1, 1.0)
    torch.cuda.synchronize()
    assert int(cache.data.count_nonzero().item()) == 0, "a refused call wrote to the cache"


def test_long_context_split_256_ways():
    w = dataclasses.replace(synth.WORKLOADS["gqa_decode"], num_kv_heads=1, num_q_heads=4, batch=1, context=262144)
    print("[limits] 262144 tokens, 1 kv head, 4 q heads", flush=True)
    worst = _step_and_check(w, [262144], 93, [0])
    print(f"  worst relative error {worst:.2e}", flush=True)
