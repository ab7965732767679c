"""GPU tests of the block transfers between the packed cache and pinned host
memory (tq_offload_blocks / tq_restore_blocks): the qiita LMCache article's
checks, in its order.

* byte round trip: the host copy and the restored blocks equal the original
  bytes (T(Q(X)) = Q(X));
* adjacent regions: host bytes outside the copied ranges, blocks of the cache
  that were not restored, and skipped ids keep their 0xA5 sentinel;
* path comparison: decode over blocks restored into other block ids (tables
  remapped) equals decode over the original cache, and both match the oracle;
* timing: t_copy ~ t0 + B / beta fitted over transfer sizes (printed).
"""
import dataclasses
import math
import time

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


def _filled_cache(w, lens, seed):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    lay = synth.paged_layout(len(lens), lens, seed, spare_blocks=5)
    total = int(sum(lens))
    k = synth.kv_tensor(w, total, "k", seed)
    v = synth.kv_tensor(w, total, "v", seed)
    slots = np.concatenate([lay.slots(b, 0, n) for b, n in enumerate(lens)])
    ctx = H.make_context(w)
    cache = PagedKVCache(ctx, lay.num_blocks, fill=0xA5)
    cache.append(H.upload(k, w, torch), H.upload(v, w, torch), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    return ctx, lay, cache


def test_round_trip_bytes_and_sentinels():
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS["gqa_decode"]
    ctx, lay, cache = _filled_cache(w, [300, 77], 51)
    bb = cache.block_bytes
    used = np.unique(lay.block_tables[lay.block_tables >= 0])
    ids = np.concatenate([used, [lay.num_blocks + 3, -1]]).astype(np.int32)     # two ids to skip
    n = len(ids)
    pad = 256
    host_all = torch.full((n * bb + 2 * pad,), 0xA5, dtype=torch.uint8, pin_memory=True)
    host = host_all[pad:pad + n * bb]
    ids_dev = torch.from_numpy(ids).cuda()
    cache.offload_blocks(ids_dev, host)
    torch.cuda.synchronize()
    src = cache.data.cpu().numpy().reshape(lay.num_blocks, bb)
    h = host_all.numpy()
    got = h[pad:pad + n * bb].reshape(n, bb)
    assert np.array_equal(got[:len(used)], src[used]), "offloaded bytes differ"
    assert np.all(got[len(used):] == 0xA5), "a skipped id wrote to the host buffer"
    assert np.all(h[:pad] == 0xA5) and np.all(h[pad + n * bb:] == 0xA5), "bytes outside the host range changed"

    # restore into other block ids of a fresh cache (a seeded permutation)
    perm = np.random.default_rng(52).permutation(lay.num_blocks).astype(np.int32)
    new_ids = np.concatenate([perm[used], [-5, lay.num_blocks]]).astype(np.int32)
    cache2 = PagedKVCache(ctx, lay.num_blocks, fill=0xA5)
    cache2.restore_blocks(host, torch.from_numpy(new_ids).cuda())
    torch.cuda.synchronize()
    dst = cache2.data.cpu().numpy().reshape(lay.num_blocks, bb)
    assert np.array_equal(dst[perm[used]], src[used]), "restored bytes differ"
    others = np.setdiff1d(np.arange(lay.num_blocks), perm[used])
    assert np.all(dst[others] == 0xA5), "a block outside the restore list changed"


def test_decode_through_host_equals_decode_in_hbm():
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    generic = dataclasses.replace(synth.WORKLOADS["qjl"], head_dim=64)      # the generic path
    for name in ("gqa_decode", "qjl", "qjl@d64"):
        w = generic if name == "qjl@d64" else synth.WORKLOADS[name]
        lens = [300, 77, 16]
        ctx, lay, cache = _filled_cache(w, lens, 53)
        used = np.unique(lay.block_tables[lay.block_tables >= 0]).astype(np.int32)
        host = torch.empty((len(used) * cache.block_bytes,), dtype=torch.uint8, pin_memory=True)
        cache.offload_blocks(torch.from_numpy(used).cuda(), host)
        perm = np.random.default_rng(54).permutation(lay.num_blocks).astype(np.int32)
        cache2 = PagedKVCache(ctx, lay.num_blocks, fill=0)
        cache2.restore_blocks(host, torch.from_numpy(perm[used]).cuda())
        tables2 = np.where(lay.block_tables >= 0, perm[np.maximum(lay.block_tables, 0)], -1).astype(np.int32)
        q = synth.query_tensor(w, len(lens), 53)
        scale = 1.0 / math.sqrt(w.head_dim)
        seq = torch.from_numpy(lay.seq_lens).cuda()
        o1 = cache.decode(H.upload(q, w, torch), torch.from_numpy(lay.block_tables).cuda(), seq, max(lens), scale)
        o2 = cache2.decode(H.upload(q, w, torch), torch.from_numpy(tables2).cuda(), seq, max(lens), scale)
        torch.cuda.synchronize()
        o1 = o1.cpu().numpy().astype(np.float64)
        o2 = o2.cpu().numpy().astype(np.float64)
        _, ref = H.oracle_decode(w, q, cache.data.cpu().numpy(), lay)
        for b in range(len(lens)):
            for hq in range(w.num_q_heads):
                assert H.rel_err(o2[b, hq], o1[b, hq]) <= 1e-5
                assert H.rel_err(o2[b, hq], ref[b, hq]) <= H.REL_TOL
        print(f"  {name}: decode through host memory matches", flush=True)


def test_unmapped_host_buffer_is_refused():
    w = synth.WORKLOADS["gqa_decode"]
    ctx, lay, cache = _filled_cache(w, [40], 55)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    plain = np.zeros(cache.block_bytes + 64, np.uint8)
    addr = (plain.ctypes.data + 15) // 16 * 16
    with pytest.raises(tq.TQError):
        ctx.offload_blocks(cache.data, cache.num_blocks, ids, 1, addr)


def test_transfer_time_model():
    """t_copy ~ t0 + B / beta over sizes from one block to 147 MB (one GQA layer)."""
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS["gqa_decode"]
    ctx = H.make_context(w)
    nb = 8192
    cache = PagedKVCache(ctx, nb, fill=0x5A)
    bb = cache.block_bytes
    host = torch.empty((nb * bb,), dtype=torch.uint8, pin_memory=True)
    ids_all = torch.from_numpy(np.random.default_rng(56).permutation(nb).astype(np.int32)).cuda()
    rows = []
    for n in (1, 16, 128, 1024, 8192):
        ids = ids_all[:n].contiguous()
        for direction in ("offload", "restore"):
            fn = (lambda: cache.offload_blocks(ids, host)) if direction == "offload" else \
                 (lambda: cache.restore_blocks(host, ids))
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            rows.append((direction, n * bb, e0.elapsed_time(e1) / reps * 1e-3))
    for direction in ("offload", "restore"):
        B = np.array([r[1] for r in rows if r[0] == direction], np.float64)
        t = np.array([r[2] for r in rows if r[0] == direction], np.float64)
        A = np.stack([np.ones_like(B), B], 1)
        (t0, inv_beta), *_ = np.linalg.lstsq(A, t, rcond=None)
        print(f"  {direction}: t0 = {t0 * 1e6:.1f} us, beta = {1 / inv_beta / 1e9:.1f} GB/s; "
              + ", ".join(f"{b / 1e6:.2f} MB in {s * 1e6:.1f} us" for b, s in zip(B, t)), flush=True)
        assert inv_beta > 0
