"""Caller-side state of the SWAN decode step: device planes of the hybrid
cache and the per-step buffers, allocated with torch (device memory only)
and handed to libswan as raw pointers.  All computation is in libswan."""
from __future__ import annotations

import torch

from . import swan as S


class HybridCache:
    """Sparse planes + dense buffer of one layer, laid out as include/swan.h
    describes (contiguous when dims.block_size == 0, else a paged pool whose
    block table the caller supplies as an int32 [B][max_blocks] tensor)."""

    def __init__(self, dims: S.swan_dims, device="cuda", block_table: torch.Tensor | None = None):
        self.dims = dims
        n_idx, n_val, n_buf = S.swan_cache_bytes(dims)
        z = lambda n, dt: torch.zeros(max(n, 1), dtype=dt, device=device)
        self.k_idx, self.v_idx = z(n_idx, torch.uint8), z(n_idx, torch.uint8)
        self.k_val, self.v_val = z(n_val // 2, torch.float16), z(n_val // 2, torch.float16)
        self.k_buf, self.v_buf = z(n_buf // 2, torch.float16), z(n_buf // 2, torch.float16)
        self.block_table = None
        if dims.block_size > 0:
            if block_table is None:
                raise ValueError("paged layout needs a block table")
            self.set_block_table(block_table)
        self._struct = None

    @property
    def k_stride(self) -> int:
        return S.swan_row_stride(self.dims.k)

    def set_block_table(self, bt: torch.Tensor):
        d = self.dims
        if bt.dtype != torch.int32 or tuple(bt.shape) != (d.B, d.max_blocks) or not bt.is_contiguous():
            raise ValueError(f"block table must be contiguous int32 [{d.B}][{d.max_blocks}]")
        self.block_table = bt
        self._struct = None

    def struct(self) -> S.swan_cache:
        if self._struct is None:
            p = lambda t: None if t is None else t.data_ptr()
            self._struct = S.swan_cache(p(self.k_idx), p(self.k_val), p(self.v_idx), p(self.v_val),
                                        p(self.k_buf), p(self.v_buf), p(self.block_table))
        return self._struct

    # shaped views (contiguous layout) for inspection
    def sparse_views(self):
        d, ks = self.dims, self.k_stride
        if d.block_size > 0:
            shp = (d.num_blocks, d.H_kv, d.block_size, ks)
        else:
            shp = (d.B, d.H_kv, d.n_cap, ks)
        n = 1
        for s in shp:
            n *= s
        return tuple(t[:n].view(shp) for t in (self.k_idx, self.k_val, self.v_idx, self.v_val))

    def buffer_views(self):
        d = self.dims
        n = d.B * d.H_kv * d.R * 128
        shp = (d.B, d.H_kv, d.R, 128)
        return self.k_buf[:n].view(shp), self.v_buf[:n].view(shp)


class SwanDecoder:
    """One layer's decode step: project -> append/evict -> decode attention,
    enqueued back to back on one stream with no host synchronisation."""

    def __init__(self, dims: S.swan_dims, P_qk: torch.Tensor, rope_base: float = 10000.0, device="cuda",
                 block_table: torch.Tensor | None = None):
        self.dims, self.P_qk, self.rope_base = dims, P_qk, float(rope_base)
        self.cache = HybridCache(dims, device, block_table)
        B, N, H = dims.B, dims.N_h, dims.H_kv
        self.q_hat = torch.empty((B, N, 128), dtype=torch.float32, device=device)
        self.k_hat = torch.empty((B, H, 128), dtype=torch.float16, device=device)
        self.o_hat = torch.empty((B, N, 128), dtype=torch.float32, device=device)
        self.workspace = torch.empty(0, dtype=torch.uint8, device=device)
        self.device = device

    def ensure_workspace(self, max_pos: int):
        need = S.swan_decode_workspace_bytes(self.dims, max_pos)
        if self.workspace.numel() < need:
            self.workspace = torch.empty(int(need * 1.25) + 256, dtype=torch.uint8, device=self.device)

    def prefill(self, length: torch.Tensor, max_len: int, k_raw: torch.Tensor, v_hat: torch.Tensor, stream=None):
        S.swan_prefill_convert(self.dims, self.cache.struct(), length, max_len, k_raw, v_hat, self.P_qk,
                               self.rope_base, stream)

    def project(self, q, k, pos, stream=None):
        S.swan_project_qk(self.dims, q, k, pos, self.P_qk, self.rope_base, self.q_hat, self.k_hat, stream)

    def append(self, pos, max_pos, v_hat, stream=None):
        S.swan_append_evict(self.dims, self.cache.struct(), pos, max_pos, self.k_hat, v_hat, stream)

    def decode(self, pos, max_pos, stream=None):
        self.ensure_workspace(max_pos)
        S.swan_decode_attn(self.dims, self.cache.struct(), pos, max_pos, self.q_hat, self.o_hat, self.workspace,
                           stream)
        return self.o_hat

    def step(self, q, k, v_hat, pos, max_pos, stream=None):
        self.project(q, k, pos, stream)
        self.append(pos, max_pos, v_hat, stream)
        return self.decode(pos, max_pos, stream)
