"""Thin ctypes binding of the C ABI in include/tq.h (argument marshalling only).

Every step of quantize-append, decode attention and dequantize runs in the HIP
kernels of libtq.so.  Device buffers are passed as anything with a
``data_ptr()`` method (torch tensors on the GPU) or as raw integer addresses;
PyTorch is used only for device memory and streams.  If libtq.so is missing,
loading fails loudly: there is no other implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

ABI_VERSION = 1
FORMAT_VERSION = 2
BLOCK_TOKENS = 16
STATIC_SCRATCH_BYTES = 65536 + 8388608     # TQ_STATIC_SCRATCH_BYTES

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE_TOO_SMALL, TQ_ERR_HIP, TQ_ERR_OUT_OF_MEMORY = range(6)
TQ_F32, TQ_BF16 = 0, 1
KEY_MODES = {"lloyd": 0, "lloyd_nc": 1, "lloyd_qjl": 2, "fp8": 3, "polar": 4}
VAL_MODES = {"uniform": 0, "lloyd": 1}

# Every entry point declared in include/tq.h.
EXPORTS = ("tq_abi_version", "tq_validate_config", "tq_layout_for_config", "tq_codebook", "tq_create",
           "tq_destroy", "tq_layout_query", "tq_quantize_append", "tq_decode_workspace_bytes",
           "tq_decode_attention", "tq_decode_attention_noalloc", "tq_append_decode", "tq_offload_blocks",
           "tq_restore_blocks", "tq_dequantize", "tq_dequantize_rows", "tq_status_string", "tq_last_error_message")


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ("abi_version", "head_dim", "num_kv_heads", "num_q_heads",
                                                "key_bits", "key_mode", "val_bits", "val_mode", "block_tokens")]


class Layout(ctypes.Structure):
    _fields_ = [("format_version", ctypes.c_uint32)] + [(n, ctypes.c_size_t) for n in (
        "page_bytes", "token_head_bytes", "off_kcodes", "row_kcodes", "off_knorm", "off_ksigns", "row_ksigns",
        "off_kresid", "off_vcodes", "row_vcodes", "off_vmin", "off_vscale")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def library() -> ctypes.CDLL:
    """Load libtq.so (built by __graft_entry__.build()); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float
    sig = {
        "tq_abi_version": (ctypes.c_int, []),
        "tq_validate_config": (ctypes.c_int, [ctypes.POINTER(Config)]),
        "tq_layout_for_config": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(Layout)]),
        "tq_codebook": (ctypes.c_int, [U32, U32, P, P]),
        "tq_create": (ctypes.c_int, [ctypes.POINTER(Config), P, P, ctypes.POINTER(P)]),
        "tq_destroy": (None, [P]),
        "tq_layout_query": (ctypes.c_int, [P, ctypes.POINTER(Layout)]),
        "tq_quantize_append": (ctypes.c_int, [P, P, P, ctypes.c_int, I64, P, P, I64, P]),
        "tq_decode_workspace_bytes": (SZ, [P, I32, I32]),
        "tq_decode_attention": (ctypes.c_int, [P, P, ctypes.c_int, P, I64, P, I32, P, I32, I32, F32, P, P, P, SZ, P]),
        "tq_decode_attention_noalloc": (ctypes.c_int, [P, P, ctypes.c_int, P, I64, P, I32, P, I32, I32, F32, P, P, P]),
        "tq_append_decode": (ctypes.c_int, [P, P, P, P, ctypes.c_int, P, I64, P, I32, P, I32, I32, F32, P, P, P,
                                            SZ, P]),
        "tq_offload_blocks": (ctypes.c_int, [P, P, I64, P, I64, P, P]),
        "tq_restore_blocks": (ctypes.c_int, [P, P, P, I64, P, I64, P]),
        "tq_dequantize": (ctypes.c_int, [P, P, I64, P, I64, P, P, P]),
        "tq_dequantize_rows": (ctypes.c_int, [P, P, I64, P, I64, P, P, P, I64, ctypes.c_int, P]),
        "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tq_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return library().tq_status_string(s).decode()


def _check(s: int):
    if s != TQ_OK:
        raise TQError(s, library().tq_last_error_message().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def make_config(head_dim=128, num_kv_heads=1, num_q_heads=1, key_bits=4, key_mode="lloyd_nc", val_bits=4,
                val_mode="uniform", block_tokens=BLOCK_TOKENS, abi_version=ABI_VERSION) -> Config:
    km = KEY_MODES[key_mode] if isinstance(key_mode, str) else int(key_mode)
    vm = VAL_MODES[val_mode] if isinstance(val_mode, str) else int(val_mode)
    return Config(abi_version, head_dim, num_kv_heads, num_q_heads, key_bits, km, val_bits, vm, block_tokens)


def validate_config(cfg: Config) -> int:
    """tq_validate_config: returns the status code (host only)."""
    return library().tq_validate_config(ctypes.byref(cfg))


def layout_for_config(cfg: Config) -> Layout:
    out = Layout()
    _check(library().tq_layout_for_config(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def codebook(bits: int, head_dim: int = 128):
    """The library's fp32 Lloyd-Max codebook (host only): (centroids, thresholds)."""
    c = np.zeros(1 << bits, np.float32)
    t = np.zeros((1 << bits) - 1, np.float32)
    _check(library().tq_codebook(bits, head_dim, c.ctypes.data, t.ctypes.data))
    return c, t


class Context:
    """tq_ctx: immutable constants (codebook, signs, S) on the current HIP device."""

    def __init__(self, cfg: Config, signs: np.ndarray, S: Optional[np.ndarray] = None):
        lib = library()
        self.cfg = cfg
        s = np.ascontiguousarray(signs, dtype=np.int8)
        Sp = None
        if S is not None:
            S = np.ascontiguousarray(S, dtype=np.float32)
            Sp = S.ctypes.data
        h = ctypes.c_void_p()
        _check(lib.tq_create(ctypes.byref(cfg), s.ctypes.data, Sp, ctypes.byref(h)))
        self._h = h
        lay = Layout()
        _check(lib.tq_layout_query(h, ctypes.byref(lay)))
        self.layout = lay

    def close(self):
        if getattr(self, "_h", None):
            library().tq_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def page_bytes(self) -> int:
        return self.layout.page_bytes

    def quantize_append(self, k, v, slot_mapping, cache, num_blocks: int, dtype: int, num_tokens: int,
                        stream=None):
        """tq_quantize_append (asynchronous on `stream`)."""
        _check(library().tq_quantize_append(self._h, _ptr(k), _ptr(v), dtype, num_tokens, _ptr(slot_mapping),
                                            _ptr(cache), num_blocks, _stream(stream)))

    def workspace_bytes(self, batch: int, max_seq_len: int) -> int:
        return int(library().tq_decode_workspace_bytes(self._h, batch, max_seq_len))

    def decode_attention(self, q, dtype: int, cache, num_blocks: int, block_tables, max_blocks_per_seq: int,
                         seq_lens, batch: int, max_seq_len: int, softmax_scale: float, out, workspace,
                         workspace_bytes: int, logits_out=None, stream=None):
        """tq_decode_attention (asynchronous on `stream`)."""
        _check(library().tq_decode_attention(self._h, _ptr(q), dtype, _ptr(cache), num_blocks, _ptr(block_tables),
                                             max_blocks_per_seq, _ptr(seq_lens), batch, max_seq_len,
                                             float(softmax_scale), _ptr(out), _ptr(logits_out), _ptr(workspace),
                                             workspace_bytes, _stream(stream)))

    def decode_attention_noalloc(self, q, dtype: int, cache, num_blocks: int, block_tables, max_blocks_per_seq: int,
                                 seq_lens, batch: int, max_seq_len: int, softmax_scale: float, out, logits_out=None,
                                 stream=None):
        """tq_decode_attention_noalloc (asynchronous on `stream`; the library's static scratch)."""
        _check(library().tq_decode_attention_noalloc(self._h, _ptr(q), dtype, _ptr(cache), num_blocks,
                                                     _ptr(block_tables), max_blocks_per_seq, _ptr(seq_lens), batch,
                                                     max_seq_len, float(softmax_scale), _ptr(out), _ptr(logits_out),
                                                     _stream(stream)))

    def append_decode(self, k_new, v_new, q, dtype: int, cache, num_blocks: int, block_tables,
                      max_blocks_per_seq: int, seq_lens, batch: int, max_seq_len: int, softmax_scale: float, out,
                      workspace, workspace_bytes: int, logits_out=None, stream=None):
        """tq_append_decode (asynchronous on `stream`)."""
        _check(library().tq_append_decode(self._h, _ptr(k_new), _ptr(v_new), _ptr(q), dtype, _ptr(cache), num_blocks,
                                          _ptr(block_tables), max_blocks_per_seq, _ptr(seq_lens), batch,
                                          max_seq_len, float(softmax_scale), _ptr(out), _ptr(logits_out),
                                          _ptr(workspace), workspace_bytes, _stream(stream)))

    def offload_blocks(self, cache, num_blocks: int, block_ids, n: int, host_dst, stream=None):
        """tq_offload_blocks (asynchronous on `stream`)."""
        _check(library().tq_offload_blocks(self._h, _ptr(cache), num_blocks, _ptr(block_ids), n, _ptr(host_dst),
                                           _stream(stream)))

    def restore_blocks(self, host_src, block_ids, n: int, cache, num_blocks: int, stream=None):
        """tq_restore_blocks (asynchronous on `stream`)."""
        _check(library().tq_restore_blocks(self._h, _ptr(host_src), _ptr(block_ids), n, _ptr(cache), num_blocks,
                                           _stream(stream)))

    def dequantize(self, cache, num_blocks: int, slots, n: int, k_out, v_out, stream=None):
        """tq_dequantize (asynchronous on `stream`)."""
        _check(library().tq_dequantize(self._h, _ptr(cache), num_blocks, _ptr(slots), n, _ptr(k_out), _ptr(v_out),
                                       _stream(stream)))

    def dequantize_rows(self, cache, num_blocks: int, slots, n: int, rows, k_buf, v_buf, buf_rows: int, out_dtype: int,
                        stream=None):
        """tq_dequantize_rows (asynchronous on `stream`); rows may be None (row i)."""
        _check(library().tq_dequantize_rows(self._h, _ptr(cache), num_blocks, _ptr(slots), n, _ptr(rows),
                                            _ptr(k_buf), _ptr(v_buf), buf_rows, out_dtype, _stream(stream)))
