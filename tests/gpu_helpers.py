"""Test-side helpers for GPU parity: move an oracle-built logical cache into
the GPU layout, read GPU planes back in logical order, and error metrics.
Inputs always flow oracle -> GPU, never the other way."""
import numpy as np
import torch

from decode_attention_compressed_02_amd import swan as S
from decode_attention_compressed_02_amd.cache import HybridCache, SwanDecoder


def rel_l2_max(got, want):
    """max over (b, head) of ||got - want||_2 / ||want||_2."""
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    num = np.linalg.norm(got - want, axis=-1)
    den = np.maximum(np.linalg.norm(want, axis=-1), 1e-300)
    return float((num / den).max())


def dims_for(oc, split_tokens=0, block_size=0, max_blocks=0, num_blocks=0):
    return S.make_dims(oc.B, oc.N_h, oc.H_kv, oc.R, oc.k, n_cap=oc.ncap if block_size == 0 else 0,
                       block_size=block_size, max_blocks=max_blocks, num_blocks=num_blocks,
                       split_tokens=split_tokens, value_format=oc.value_format,
                       k_v=oc.k_v if oc.k_v != oc.k else 0)


def value_storage(v, value_format):
    """Stored form of oracle values (float64, exact in the format): fp16, or
    E4M3 bytes (torch's float8_e4m3fn conversion is exact on E4M3 values)."""
    if value_format == S.SWAN_VALUES_FP8_E4M3:
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy()
    return np.asarray(v).astype(np.float16)


def assert_values_bits(stored, oracle_vals, value_format):
    """Stored values equal, bit for bit (sign of zero included), to the
    oracle's values in the same format."""
    want = value_storage(oracle_vals, value_format)
    view = np.uint8 if value_format == S.SWAN_VALUES_FP8_E4M3 else np.uint16
    np.testing.assert_array_equal(np.ascontiguousarray(stored).view(view), np.ascontiguousarray(want).view(view))


def value_f64(stored, value_format):
    """Stored values (fp16, or E4M3 bytes) as float64."""
    if value_format == S.SWAN_VALUES_FP8_E4M3:
        t = torch.from_numpy(np.ascontiguousarray(stored, np.uint8)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    return np.asarray(stored).astype(np.float64)


def upload(cache: HybridCache, oc, block_table: np.ndarray | None = None, rows=None):
    """Write the oracle state `oc` (logical rows) into the GPU planes.  In the
    paged layout only rows < rows[b] of sequence b are written (default: all
    ncap), so that a short sequence sharing blocks with a longer one does not
    overwrite the longer one's rows."""
    d = cache.dims
    planes = cache.sparse_views()
    src = (oc.kidx, value_storage(oc.kval, d.value_format), oc.vidx, value_storage(oc.vval, d.value_format))
    for dst, s in zip(planes, src):
        k = s.shape[-1]  # kept entries of this plane (k or k_v)
        host = np.zeros(tuple(dst.shape), dtype=s.dtype)
        if d.block_size == 0:
            host[:, :, :oc.ncap, :k] = s
        else:
            bs = d.block_size
            for b in range(oc.B):
                for r in range(oc.ncap if rows is None else rows[b]):
                    blk = block_table[b, r // bs]
                    if blk >= 0:
                        host[blk, :, r % bs, :k] = s[b, :, r]
        dst.copy_(torch.from_numpy(host))
    if d.R > 0:
        kb, vb = cache.buffer_views()
        kb.copy_(torch.from_numpy(oc.ringk.astype(np.float16)))
        vb.copy_(torch.from_numpy(oc.ringv.astype(np.float16)))


def download_rows(cache: HybridCache, B, H, n_rows, block_table=None):
    """GPU sparse planes in logical order: 4 arrays [B][H][n_rows][k_stride]."""
    d = cache.dims
    planes = [p.cpu().numpy() for p in cache.sparse_views()]
    if d.block_size == 0:
        return [p[:, :, :n_rows] for p in planes]
    bs = d.block_size
    out = [np.zeros((B, H, n_rows, p.shape[-1]), p.dtype) for p in planes]
    for b in range(B):
        for r in range(n_rows):
            blk = block_table[b, r // bs]
            for o, p in zip(out, planes):
                o[b, :, r] = p[blk, :, r % bs]
    return out


def make_decoder(oc, P32, rope_base=10000.0, **dim_kw):
    bt = dim_kw.pop("block_table", None)
    d = dims_for(oc, **dim_kw)
    dec = SwanDecoder(d, torch.from_numpy(np.ascontiguousarray(P32)).cuda(), rope_base,
                      block_table=None if bt is None else torch.from_numpy(bt.astype(np.int32)).cuda())
    return dec
