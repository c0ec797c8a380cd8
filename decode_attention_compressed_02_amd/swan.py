"""Python binding of libswan (include/swan.h): argument marshalling only.

Every function has the name of its C entry point and takes torch tensors for
the device arrays (PyTorch supplies device memory and streams; every step of
the computation runs in the HIP kernels of libswan).  A non-OK status raises
SwanError with the library's message.  The binding fails loudly when the
library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libswan.so")

SWAN_OK, SWAN_ERR_INVALID_ARG, SWAN_ERR_UNSUPPORTED, SWAN_ERR_CAPACITY, SWAN_ERR_HIP = range(5)

EXPORTS = ("swan_status_str", "swan_last_error", "swan_row_stride", "swan_cache_bytes", "swan_project_qk",
           "swan_append_evict", "swan_decode_workspace_bytes", "swan_decode_num_splits", "swan_decode_attn",
           "swan_decode_split", "swan_decode_reduce", "swan_prefill_convert", "swan_copy_blocks",
           "swan_project_append", "swan_paged_update", "swan_project_append_paged",
           "swan_measure_stream_read", "swan_decode_attn_noalloc", "swan_measure_mfma_f64")


class SwanError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class swan_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "N_h", "H_kv", "d_h", "R", "k", "n_cap", "block_size", "max_blocks",
                                         "num_blocks", "split_tokens", "value_format", "k_v", "layers")]

    def __repr__(self):
        return "swan_dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class swan_cache(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("k_idx", "k_val", "v_idx", "v_val", "k_buf", "v_buf", "block_table")]


_lib = None


def lib():
    """The loaded libswan (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc for gfx950); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        P, V, I32, I64, F, SZ = C.POINTER, C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        D, Cc = P(swan_dims), P(swan_cache)
        sig = {
            "swan_status_str": ([C.c_int], C.c_char_p),
            "swan_last_error": ([], C.c_char_p),
            "swan_row_stride": ([I32], I32),
            "swan_cache_bytes": ([D, P(SZ)], C.c_int),
            "swan_project_qk": ([D, V, V, V, V, F, V, V, V], C.c_int),
            "swan_append_evict": ([D, Cc, V, I32, V, V, V], C.c_int),
            "swan_project_append": ([D, Cc, V, V, V, V, I32, V, F, V, V, V], C.c_int),
            "swan_decode_workspace_bytes": ([D, I32], SZ),
            "swan_decode_num_splits": ([D, I32], I32),
            "swan_decode_attn": ([D, Cc, V, I32, V, V, V, SZ, V], C.c_int),
            "swan_decode_split": ([D, Cc, V, I32, V, V, SZ, V], C.c_int),
            "swan_decode_reduce": ([D, V, I32, V, SZ, V, V], C.c_int),
            "swan_prefill_convert": ([D, Cc, V, I32, I64, V, V, V, F, V], C.c_int),
            "swan_copy_blocks": ([D, Cc, V, V, I32, V], C.c_int),
            "swan_paged_update": ([D, Cc, V, V, I32, V, I32, V], C.c_int),
            "swan_project_append_paged": ([D, Cc, V, V, V, V, I32, V, F, V, V, V, V, I32, V, I32, V], C.c_int),
            "swan_measure_stream_read": ([V, SZ, I32, V, V], C.c_int),
            "swan_decode_attn_noalloc": ([D, Cc, V, I32, V, V, V], C.c_int),
            "swan_measure_mfma_f64": ([C.c_double, I32, I32, V, V], C.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


def _check(status: int):
    if status != SWAN_OK:
        L = lib()
        raise SwanError(status, f"{L.swan_status_str(status).decode()}: {L.swan_last_error().decode()}")


def _ptr(t, dtype=None, name="array"):
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(getattr(stream, "cuda_stream", stream))


SWAN_VALUES_FP16, SWAN_VALUES_FP8_E4M3 = 0, 1


def make_dims(B, N_h, H_kv, R, k, n_cap=0, d_h=128, block_size=0, max_blocks=0, num_blocks=0, split_tokens=0,
              value_format=SWAN_VALUES_FP16, k_v=0, layers=0):
    return swan_dims(B, N_h, H_kv, d_h, R, k, n_cap, block_size, max_blocks, num_blocks, split_tokens, value_format,
                     k_v, layers)


def swan_row_stride(k: int) -> int:
    return int(lib().swan_row_stride(k))


def swan_cache_bytes(dims: swan_dims):
    """(k_idx, k_val, v_idx, v_val, k_buf = v_buf) bytes."""
    out = (C.c_size_t * 5)()
    _check(lib().swan_cache_bytes(C.byref(dims), out))
    return tuple(int(x) for x in out)


def swan_decode_workspace_bytes(dims: swan_dims, max_pos: int) -> int:
    return int(lib().swan_decode_workspace_bytes(C.byref(dims), int(max_pos)))


def swan_decode_num_splits(dims: swan_dims, max_pos: int) -> int:
    return int(lib().swan_decode_num_splits(C.byref(dims), int(max_pos)))


def swan_project_qk(dims, q, k, pos, P_qk, rope_base, q_hat, k_hat, stream=None):
    import torch
    _check(lib().swan_project_qk(C.byref(dims), _ptr(q, torch.float32, "q"), _ptr(k, torch.float32, "k"),
                                 _ptr(pos, torch.int32, "pos"), _ptr(P_qk, torch.float32, "P_qk"), float(rope_base),
                                 _ptr(q_hat, torch.float32, "q_hat"), _ptr(k_hat, torch.float16, "k_hat"),
                                 _stream(stream)))


def swan_project_append(dims, cache: "swan_cache", q, k, v_hat, pos, max_pos, P_qk, rope_base, q_hat, k_hat,
                        stream=None):
    import torch
    _check(lib().swan_project_append(C.byref(dims), C.byref(cache), _ptr(q, torch.float32, "q"),
                                     _ptr(k, torch.float32, "k"), _ptr(v_hat, torch.float32, "v_hat"),
                                     _ptr(pos, torch.int32, "pos"), int(max_pos), _ptr(P_qk, torch.float32, "P_qk"),
                                     float(rope_base), _ptr(q_hat, torch.float32, "q_hat"),
                                     _ptr(k_hat, torch.float16, "k_hat"), _stream(stream)))


def swan_append_evict(dims, cache: "swan_cache", pos, max_pos, k_hat, v_hat, stream=None):
    import torch
    _check(lib().swan_append_evict(C.byref(dims), C.byref(cache), _ptr(pos, torch.int32, "pos"), int(max_pos),
                                   _ptr(k_hat, torch.float16, "k_hat"), _ptr(v_hat, torch.float32, "v_hat"),
                                   _stream(stream)))


def swan_decode_attn(dims, cache, pos, max_pos, q_hat, o_hat, workspace, stream=None):
    import torch
    _check(lib().swan_decode_attn(C.byref(dims), C.byref(cache), _ptr(pos, torch.int32, "pos"), int(max_pos),
                                  _ptr(q_hat, torch.float32, "q_hat"), _ptr(o_hat, torch.float32, "o_hat"),
                                  _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))


def swan_decode_attn_noalloc(dims, cache, pos, max_pos, q_hat, o_hat, stream=None):
    """swan_decode_attn over the library's per-GPU scratch array: no workspace argument."""
    import torch
    _check(lib().swan_decode_attn_noalloc(C.byref(dims), C.byref(cache), _ptr(pos, torch.int32, "pos"), int(max_pos),
                                          _ptr(q_hat, torch.float32, "q_hat"), _ptr(o_hat, torch.float32, "o_hat"),
                                          _stream(stream)))


def swan_decode_split(dims, cache, pos, max_pos, q_hat, workspace, stream=None):
    import torch
    _check(lib().swan_decode_split(C.byref(dims), C.byref(cache), _ptr(pos, torch.int32, "pos"), int(max_pos),
                                   _ptr(q_hat, torch.float32, "q_hat"), _ptr(workspace, None, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def swan_decode_reduce(dims, pos, max_pos, workspace, o_hat, stream=None):
    import torch
    _check(lib().swan_decode_reduce(C.byref(dims), _ptr(pos, torch.int32, "pos"), int(max_pos),
                                    _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                    _ptr(o_hat, torch.float32, "o_hat"), _stream(stream)))


def swan_prefill_convert(dims, cache, length, max_len, k_raw, v_hat, P_qk, rope_base, stream=None):
    import torch
    T_stride = k_raw.shape[2]
    if v_hat.shape != k_raw.shape:
        raise ValueError("k_raw and v_hat must have the same shape [B][H_kv][T][128]")
    _check(lib().swan_prefill_convert(C.byref(dims), C.byref(cache), _ptr(length, torch.int32, "len"), int(max_len),
                                      int(T_stride), _ptr(k_raw, torch.float32, "k_raw"),
                                      _ptr(v_hat, torch.float32, "v_hat"), _ptr(P_qk, torch.float32, "P_qk"),
                                      float(rope_base), _stream(stream)))


def swan_copy_blocks(dims, cache, src, dst, stream=None):
    """Copy paged blocks src[i] -> dst[i] (int32 device tensors of equal length)."""
    import torch
    if src.numel() != dst.numel():
        raise ValueError("src and dst must have the same length")
    _check(lib().swan_copy_blocks(C.byref(dims), C.byref(cache), _ptr(src, torch.int32, "src"),
                                  _ptr(dst, torch.int32, "dst"), int(src.numel()), _stream(stream)))


def _host_pairs(a, what, width=2):
    import numpy as np
    a = (np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1, width)) if a is not None
         else np.zeros((0, width), np.int32))
    if a.ndim != 2 or a.shape[1] != width:
        raise ValueError(f"{what} must be rows of {width}")
    return a


def swan_paged_update(dims, cache, block_table, entries=None, copies=None, stream=None):
    """Block-table writes (entries: host pairs (b * max_blocks + j, id)) and
    copy-on-write copies (copies: host pairs (src, dst)) carried by value in
    the launch arguments; block_table is the cache's device table."""
    import torch
    e, c = _host_pairs(entries, "entries"), _host_pairs(copies, "copies")
    _check(lib().swan_paged_update(C.byref(dims), C.byref(cache), _ptr(block_table, torch.int32, "block_table"),
                                   e.ctypes.data_as(C.c_void_p), int(e.shape[0]), c.ctypes.data_as(C.c_void_p),
                                   int(c.shape[0]), _stream(stream)))


def swan_project_append_paged(dims, cache, q, k, v_hat, pos, max_pos, P_qk, rope_base, q_hat, k_hat, block_table,
                              entries=None, copies=None, stream=None):
    """Projection, append and the paged table update of a step in one launch:
    entries are host pairs (b * max_blocks + j, id), copies host triples
    (src, dst, skip row)."""
    import torch
    e, c = _host_pairs(entries, "entries"), _host_pairs(copies, "copies", 3)
    _check(lib().swan_project_append_paged(C.byref(dims), C.byref(cache), _ptr(q, torch.float32, "q"),
                                           _ptr(k, torch.float32, "k"), _ptr(v_hat, torch.float32, "v_hat"),
                                           _ptr(pos, torch.int32, "pos"), int(max_pos),
                                           _ptr(P_qk, torch.float32, "P_qk"), float(rope_base),
                                           _ptr(q_hat, torch.float32, "q_hat"), _ptr(k_hat, torch.float16, "k_hat"),
                                           _ptr(block_table, torch.int32, "block_table"),
                                           e.ctypes.data_as(C.c_void_p), int(e.shape[0]), c.ctypes.data_as(C.c_void_p),
                                           int(c.shape[0]), _stream(stream)))


def swan_measure_stream_read(buf, waves, sink, stream=None):
    """Streaming read of the whole of `buf` (a contiguous device tensor whose
    byte size is a multiple of 16) by `waves` one-wave workgroups; sink is a
    uint32-sized device tensor of at least waves * 64 elements."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < waves * 64 * 4:
        raise ValueError("sink must hold waves * 64 uint32 words")
    _check(lib().swan_measure_stream_read(_ptr(buf, None, "buf"), nbytes, int(waves), _ptr(sink, None, "sink"),
                                          _stream(stream)))


def swan_measure_mfma_f64(x, waves, iters, sink, stream=None):
    """`waves` waves (workgroups of four) of `iters` rounds of eight fp64 16x16x4
    matrix products each (16384 flops a wave a round); sink is a float64
    device tensor of at least waves * 64 elements."""
    import torch
    if sink.numel() < waves * 64:
        raise ValueError("sink must hold waves * 64 doubles")
    _check(lib().swan_measure_mfma_f64(float(x), int(waves), int(iters), _ptr(sink, torch.float64, "sink"),
                                       _stream(stream)))
