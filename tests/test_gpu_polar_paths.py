"""GPU test: the two PolarQuant append paths write the same bytes.

Appends of at most 32768 (token, head) rows take one wave per row (keys and
values in one launch); larger ones take one lane per row (a keys kernel and a
values kernel).  Both compute every angle, radius and code with the same fp32
operations in the same order, so a cache built by one large append and one
built by chunks of the same rows must be byte-identical, for bf16 and fp32
inputs.  The values of both paths are also checked against the oracle's
quantization of the same rows (codes bit-exact outside the 1e-6 band, scalars
to their rounding tolerance).
"""
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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wave_and_lane_paths_write_the_same_bytes(dtype):
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache
    w = synth.WORKLOADS["polar3"]
    n = 4200                                   # x 8 heads = 33600 rows: above the one-wave-per-row limit
    print(f"[polar paths] {dtype}: {n} tokens x {w.num_kv_heads} heads", flush=True)
    lay = synth.paged_layout(1, [n], 81)
    slots = lay.slots(0, 0, n).astype(np.int64)
    k = synth.kv_tensor(w, n, "k", 81)
    v = synth.kv_tensor(w, n, "v", 81)
    if dtype == "f32":                          # the same values, widened
        kd = torch.from_numpy(synth.bf16_bits_to_f32(k)).cuda()
        vd = torch.from_numpy(synth.bf16_bits_to_f32(v)).cuda()
    else:
        kd, vd = H.upload(k, w, torch), H.upload(v, w, torch)
    ctx = H.make_context(w)
    whole = PagedKVCache(ctx, lay.num_blocks, fill=0)
    whole.append(kd, vd, torch.from_numpy(slots).cuda())
    chunks = PagedKVCache(ctx, lay.num_blocks, fill=0)
    for c0 in range(0, n, 1000):               # 8000 rows per call: one wave per row
        c1 = min(c0 + 1000, n)
        chunks.append(kd[c0:c1].contiguous(), vd[c0:c1].contiguous(), torch.from_numpy(slots[c0:c1]).cuda())
    torch.cuda.synchronize()
    a, b = whole.data.cpu().numpy(), chunks.data.cpu().numpy()
    diff = int(np.count_nonzero(a != b))
    assert diff == 0, f"{diff} bytes differ between the two append paths"
    # both against the oracle's quantization of the rows
    report = {}
    H.compare_append(w, a, slots, H.oracle_quantize(w, k, v), report)
    print(f"  whole append == chunked appends; vs oracle: {report}", flush=True)
