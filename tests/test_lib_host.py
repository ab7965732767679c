"""Host-side checks of the C-ABI library (no GPU): the header is plain C, the
library loads, exports every entry point that include/tq.h declares, validates
configurations, reports the page layout of the format, and builds the same fp32
codebook as the oracle."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from kv_cache_vector_randomized_amd import tq
from oracle import tq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "tq.h"\nint main(void) { return tq_abi_version() > 0 ? 0 : 1; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include", str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tq.library()
    declared = _declared_functions()
    assert set(declared) == set(tq.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.tq_abi_version() == tq.ABI_VERSION


def test_status_strings():
    for s in range(6):
        assert tq.status_string(s).startswith("TQ_")


@pytest.mark.parametrize("kw,expect", [
    (dict(), tq.TQ_OK),
    (dict(num_kv_heads=8, num_q_heads=32), tq.TQ_OK),
    (dict(num_kv_heads=8, num_q_heads=12), tq.TQ_ERR_INVALID_ARG),
    (dict(num_kv_heads=2, num_q_heads=16), tq.TQ_OK),                # group 8: tuned, two sub-groups of 4
    (dict(num_kv_heads=1, num_q_heads=3), tq.TQ_OK),                 # group 3: tuned, one head group of 3
    (dict(num_kv_heads=1, num_q_heads=16), tq.TQ_OK),
    (dict(num_kv_heads=1, num_q_heads=17), tq.TQ_ERR_UNSUPPORTED),   # more than 16 q heads per KV head
    (dict(head_dim=96), tq.TQ_ERR_INVALID_ARG),
    (dict(head_dim=64), tq.TQ_OK),
    (dict(head_dim=256), tq.TQ_OK),
    (dict(head_dim=256, key_bits=8, key_mode="lloyd_nc"), tq.TQ_OK),
    (dict(head_dim=256, key_bits=2, key_mode="lloyd_qjl", val_mode="lloyd"), tq.TQ_OK),
    (dict(head_dim=32), tq.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=512), tq.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=64, key_bits=8, key_mode="fp8"), tq.TQ_OK),                 # FP8 keys on the generic path
    (dict(num_kv_heads=1, num_q_heads=8, key_bits=8, key_mode="fp8"), tq.TQ_OK),
    (dict(head_dim=256, key_bits=3, key_mode="polar"), tq.TQ_ERR_UNSUPPORTED),  # polar: head_dim 128 only
    (dict(num_kv_heads=1, num_q_heads=8, key_bits=3, key_mode="polar"), tq.TQ_OK),
    (dict(num_kv_heads=1, num_q_heads=7, key_bits=3, key_mode="polar"), tq.TQ_OK),
    (dict(key_bits=0), tq.TQ_ERR_INVALID_ARG),
    (dict(key_bits=8), tq.TQ_OK),                    # 8-bit Lloyd-Max keys
    (dict(key_bits=5), tq.TQ_ERR_UNSUPPORTED),
    (dict(key_bits=3, key_mode="polar"), tq.TQ_OK),
    (dict(key_bits=8, key_mode="polar"), tq.TQ_ERR_UNSUPPORTED),
    (dict(key_bits=3, key_mode="polar", val_mode="lloyd"), tq.TQ_ERR_UNSUPPORTED),
    (dict(val_bits=1), tq.TQ_ERR_UNSUPPORTED),
    (dict(key_mode=3), tq.TQ_ERR_INVALID_ARG),
    (dict(val_mode=2), tq.TQ_ERR_INVALID_ARG),
    (dict(block_tokens=32), tq.TQ_ERR_INVALID_ARG),
    (dict(abi_version=2), tq.TQ_ERR_INVALID_ARG),
    (dict(key_bits=8, key_mode="fp8"), tq.TQ_OK),
    (dict(key_bits=4, key_mode="fp8"), tq.TQ_ERR_INVALID_ARG),
    (dict(key_bits=8, key_mode="fp8", val_mode="lloyd"), tq.TQ_ERR_UNSUPPORTED),
    (dict(key_mode=5), tq.TQ_ERR_INVALID_ARG),
    (dict(key_bits=8, key_mode="lloyd_nc", val_bits=3), tq.TQ_OK),
    (dict(key_bits=8, key_mode="lloyd_qjl"), tq.TQ_ERR_UNSUPPORTED),
    (dict(key_bits=6), tq.TQ_ERR_UNSUPPORTED),
])
def test_validate_config(kw, expect):
    assert tq.validate_config(tq.make_config(**kw)) == expect


def test_null_config_and_context():
    lib = tq.library()
    assert lib.tq_validate_config(None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize_append(None, None, None, 1, 1, None, None, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_decode_workspace_bytes(None, 1, 1) == 0
    assert lib.tq_destroy(None) is None
    assert b"ctx" in lib.tq_last_error_message() or lib.tq_last_error_message()


def test_every_call_refuses_a_null_context():
    """Argument errors come back synchronously as TQ_ERR_INVALID_ARG (no GPU is touched)."""
    lib = tq.library()
    calls = {
        "tq_decode_attention": (None, None, 1, None, 1, None, 1, None, 1, 1, 1.0, None, None, None, 0, None),
        "tq_append_decode": (None, None, None, None, 1, None, 1, None, 1, None, 1, 1, 1.0, None, None, None, 0, None),
        "tq_offload_blocks": (None, None, 1, None, 1, None, None),
        "tq_restore_blocks": (None, None, None, 1, None, 1, None),
        "tq_dequantize": (None, None, 1, None, 1, None, None, None),
        "tq_dequantize_rows": (None, None, 1, None, 1, None, None, None, 1, tq.TQ_BF16, None),
        "tq_layout_query": (None, None),
    }
    for name, args in calls.items():
        assert getattr(lib, name)(*args) == tq.TQ_ERR_INVALID_ARG, name
        assert b"null" in lib.tq_last_error_message(), name


@pytest.mark.parametrize("d,kb,km,vb,vm", [(128, 4, "lloyd", 4, "lloyd"), (128, 4, "lloyd_nc", 4, "uniform"),
                                           (128, 3, "lloyd_nc", 3, "uniform"), (128, 2, "lloyd_qjl", 4, "uniform"),
                                           (128, 2, "lloyd", 2, "uniform"), (128, 3, "lloyd_qjl", 3, "lloyd"),
                                           (128, 8, "fp8", 4, "uniform"), (128, 8, "fp8", 3, "uniform"),
                                           (128, 8, "lloyd_nc", 3, "uniform"), (128, 3, "polar", 4, "uniform"),
                                           (64, 3, "lloyd_qjl", 3, "uniform"), (64, 4, "lloyd_nc", 2, "lloyd"),
                                           (256, 8, "lloyd_nc", 4, "uniform"), (256, 2, "lloyd_qjl", 4, "lloyd")])
def test_layout_matches_format(d, kb, km, vb, vm):
    lay = tq.layout_for_config(tq.make_config(d, 8, 32, kb, km, vb, vm)).as_dict()
    f = O.page_fields(O.Config(d, 8, 32, kb, km, vb, vm))
    none = (1 << 64) - 1
    assert lay["format_version"] == O.FORMAT_VERSION
    assert lay["page_bytes"] == O.page_bytes(O.Config(d, 8, 32, kb, km, vb, vm))
    assert lay["token_head_bytes"] * 16 == lay["page_bytes"]
    assert (lay["off_kcodes"], lay["row_kcodes"]) == f["kcodes"]
    assert lay["off_knorm"] == (f["knorm"][0] if km != "fp8" else none)
    assert (lay["off_vcodes"], lay["row_vcodes"]) == f["vcodes"]
    if km == "lloyd_qjl":
        assert (lay["off_ksigns"], lay["row_ksigns"]) == f["ksigns"]
        assert lay["off_kresid"] == f["kres"][0]
    else:
        assert lay["off_ksigns"] == none and lay["off_kresid"] == none
    if vm == "uniform":
        assert lay["off_vmin"] == f["vmin"][0] and lay["off_vscale"] == f["vscale"][0]
    else:
        assert lay["off_vmin"] == f["vnorm"][0] and lay["off_vscale"] == none


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
def test_library_codebook_equals_oracle_rounded(bits):
    """The library solves Lloyd-Max on its own (C++, long double); its fp32 tables must be the
    fp32 rounding of the oracle's fp64 solution (at most 1 ulp apart)."""
    c, t = tq.codebook(bits, 128)
    cb = O.codebook(bits, 128)
    c_ref = cb.centroids.astype(np.float32)
    t_ref = cb.thresholds.astype(np.float32)
    ulp_c = np.abs(c.view(np.int32).astype(np.int64) - c_ref.view(np.int32).astype(np.int64))
    ulp_t = np.abs(t.view(np.int32).astype(np.int64) - t_ref.view(np.int32).astype(np.int64))
    assert ulp_c.max() <= 1 and ulp_t.max() <= 1, (ulp_c, ulp_t)
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    assert t[len(t) // 2] == 0.0
