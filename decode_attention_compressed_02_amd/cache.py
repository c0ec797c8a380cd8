"""Caller-side state of the SWAN decode step: device planes of the hybrid
cache and the per-step buffers, allocated with torch (device memory only)
and handed to libswan as raw pointers.  All computation is in libswan."""
from __future__ import annotations

import numpy as np
import torch

from . import swan as S


class HybridCache:
    """Sparse planes + dense buffer of one layer, laid out as include/swan.h
    describes (contiguous when dims.block_size == 0, else a paged pool whose
    block table the caller supplies as an int32 [B][max_blocks] tensor)."""

    def __init__(self, dims: S.swan_dims, device="cuda", block_table: torch.Tensor | None = None):
        self.dims = dims
        n_kidx, n_kval, n_vidx, n_vval, n_buf = S.swan_cache_bytes(dims)
        z = lambda n, dt: torch.zeros(max(n, 1), dtype=dt, device=device)
        self.k_idx, self.v_idx = z(n_kidx, torch.uint8), z(n_vidx, torch.uint8)
        # sparse values: fp16, or E4M3 bytes (held as uint8: torch has no arithmetic on them here)
        vdt, vb = (torch.uint8, 1) if dims.value_format == S.SWAN_VALUES_FP8_E4M3 else (torch.float16, 2)
        self.k_val, self.v_val = z(n_kval // vb, vdt), z(n_vval // vb, vdt)
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

    @property
    def v_stride(self) -> int:
        return S.swan_row_stride(self.dims.k_v or self.dims.k)

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

    def sub_struct(self, b0: int) -> S.swan_cache:
        """The planes as seen by a batch starting at sequence b0 (the layers of
        a multi-layer batch one at a time): contiguous planes and the dense
        buffers offset to sequence b0; a paged pool is shared by all
        sequences, so only its block table is offset (to row b0)."""
        d, base = self.dims, self.struct()
        ring = b0 * d.H_kv * d.R * 128 * 2
        if d.block_size > 0:
            return S.swan_cache(base.k_idx, base.k_val, base.v_idx, base.v_val, base.k_buf + ring,
                                base.v_buf + ring, base.block_table + b0 * d.max_blocks * 4)
        vb = 1 if d.value_format == S.SWAN_VALUES_FP8_E4M3 else 2
        rows = b0 * d.H_kv * d.n_cap
        return S.swan_cache(base.k_idx + rows * self.k_stride, base.k_val + rows * self.k_stride * vb,
                            base.v_idx + rows * self.v_stride, base.v_val + rows * self.v_stride * vb,
                            base.k_buf + ring, base.v_buf + ring, None)

    # shaped views for inspection: (k_idx, k_val, v_idx, v_val), rows of the
    # key and the value stride
    def sparse_views(self):
        d = self.dims
        lead = (d.num_blocks, d.H_kv, d.block_size) if d.block_size > 0 else (d.B, d.H_kv, d.n_cap)
        out = []
        for t, ks in ((self.k_idx, self.k_stride), (self.k_val, self.k_stride), (self.v_idx, self.v_stride),
                      (self.v_val, self.v_stride)):
            shp = lead + (ks,)
            n = 1
            for x in shp:
                n *= x
            out.append(t[:n].view(shp))
        return tuple(out)

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

    def project_append(self, q, k, v_hat, pos, max_pos, stream=None):
        S.swan_project_append(self.dims, self.cache.struct(), q, k, v_hat, pos, max_pos, self.P_qk, self.rope_base,
                              self.q_hat, self.k_hat, stream)

    def decode(self, pos, max_pos, stream=None):
        self.ensure_workspace(max_pos)
        S.swan_decode_attn(self.dims, self.cache.struct(), pos, max_pos, self.q_hat, self.o_hat, self.workspace,
                           stream)
        return self.o_hat

    def step(self, q, k, v_hat, pos, max_pos, stream=None):
        self.project_append(q, k, v_hat, pos, max_pos, stream)
        return self.decode(pos, max_pos, stream)


class StepGraph:
    """One decode step of `dec` (swan_project_append, then swan_decode_attn)
    captured as a HIP graph over fixed device buffers: replay() reissues the
    step's launches with one call and no per-launch host work.

    Before each replay the caller writes the step's inputs into the buffers
    given at capture (.q, .k, .v_hat, .pos); the output is dec.o_hat.  The
    launches keep the arguments of the capture, including the work plan and
    workspace sized for positions up to max_pos: every replayed position must
    stay within max_pos and the cache's capacity (the host checks ran once,
    at capture).  A paged decoder's host bookkeeping (prepare_step) runs
    eagerly before each replay; it writes the device table by value, so the
    graph sees the new blocks.  Nothing in the captured launches allocates
    or clears memory."""

    def __init__(self, dec: "SwanDecoder", q, k, v_hat, pos, max_pos: int):
        self.dec, self.q, self.k, self.v_hat, self.pos, self.max_pos = dec, q, k, v_hat, pos, int(max_pos)
        dec.ensure_workspace(self.max_pos)  # outside the capture: the replays never allocate
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            dec.project_append(q, k, v_hat, pos, self.max_pos)
            dec.decode(pos, self.max_pos)

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.dec.o_hat


class PoolExhausted(RuntimeError):
    """The paged pool has no free block left."""


class PagedPool:
    """Host bookkeeping of a paged sparse pool ("Reuse, Evict, or Limit
    Earlier Context" sections 1.2-1.4): physical blocks handed out from a free
    list, a reference count per block (0 free, 1 owned by one sequence, > 1
    shared and read-only), and one block table per sequence mapping logical
    block t // block_size to a physical block (-1 = not mapped).

    A write into a shared block is preceded by copy-on-write: a fresh block is
    taken from the free list, the old block's count drops by one, and the
    writer's table points to the fresh block; the caller copies the bytes
    (swan_copy_blocks) before the write."""

    def __init__(self, num_blocks: int, B: int, max_blocks: int, block_size: int, order=None):
        self.num_blocks, self.B, self.max_blocks, self.block_size = num_blocks, B, max_blocks, block_size
        self.ref = np.zeros(num_blocks, np.int32)
        order = np.arange(num_blocks) if order is None else np.asarray(order)
        if sorted(order.tolist()) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the pool's block ids")
        self._free = [int(x) for x in order[::-1]]  # pop() hands out order[0] first
        self.table = np.full((B, max_blocks), -1, np.int32)
        self.version = 0  # bumped whenever a table entry changes
        self._dirty = []  # flat table slots changed since the last take_dirty()

    @property
    def free_blocks(self) -> int:
        return len(self._free)

    def alloc(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        blk = self._free.pop()
        assert self.ref[blk] == 0
        self.ref[blk] = 1
        return blk

    def _decref(self, blk: int):
        self.ref[blk] -= 1
        assert self.ref[blk] >= 0
        if self.ref[blk] == 0:
            self._free.append(int(blk))

    def map_new(self, b: int, logical: int) -> int:
        """Give sequence b a fresh block for logical block `logical`."""
        if self.table[b, logical] >= 0:
            raise ValueError(f"logical block {logical} of sequence {b} is already mapped")
        blk = self.alloc()
        self.table[b, logical] = blk
        self._dirty.append(b * self.max_blocks + logical)
        self.version += 1
        return blk

    def share(self, src: int, dst: int, nblocks: int):
        """Map logical blocks 0..nblocks-1 of sequence dst to the physical
        blocks of sequence src (a shared prefix); their counts go up."""
        for lb in range(nblocks):
            blk = int(self.table[src, lb])
            if blk < 0:
                raise ValueError(f"logical block {lb} of sequence {src} is not mapped")
            if self.table[dst, lb] >= 0:
                raise ValueError(f"logical block {lb} of sequence {dst} is already mapped")
            self.table[dst, lb] = blk
            self.ref[blk] += 1
            self._dirty.append(dst * self.max_blocks + lb)
        self.version += 1

    def prepare_write(self, b: int, row: int):
        """Make sparse row `row` of sequence b writable.  Returns (src, dst)
        when a copy-on-write is needed (the caller must copy block src to dst
        before writing), else None."""
        lb = row // self.block_size
        if lb >= self.max_blocks:
            raise PoolExhausted(f"row {row} is past the block table ({self.max_blocks} blocks)")
        blk = int(self.table[b, lb])
        if blk < 0:
            self.map_new(b, lb)
            return None
        if self.ref[blk] == 1:
            return None
        new = self.alloc()  # may raise before anything changed
        self._decref(blk)
        self.table[b, lb] = new
        self._dirty.append(b * self.max_blocks + lb)
        self.version += 1
        return blk, new

    def release(self, b: int):
        """Sequence b finished: drop its references; blocks nobody holds return
        to the free list."""
        for lb in range(self.max_blocks):
            blk = int(self.table[b, lb])
            if blk >= 0:
                self._decref(blk)
                self.table[b, lb] = -1
                self._dirty.append(b * self.max_blocks + lb)
        self.version += 1

    def dirty_count(self) -> int:
        """Table slot changes recorded since the last take_dirty() (a slot
        changed twice counts twice)."""
        return len(self._dirty)

    def take_dirty(self):
        """(slot, block id) pairs of the table entries changed since the last
        call, slot = b * max_blocks + logical block; clears the record."""
        if not self._dirty:
            return np.zeros((0, 2), np.int32)
        slots = np.unique(np.asarray(self._dirty, np.int64))
        self._dirty = []
        return np.stack([slots, self.table.reshape(-1)[slots]], axis=1).astype(np.int32)


class PagedSwanDecoder(SwanDecoder):
    """SwanDecoder over a paged pool: before each step the rows the step will
    append are made writable (block allocation or copy-on-write), and the
    copies and changed table entries reach the device by value through
    swan_paged_update; then project -> append/evict -> decode as usual."""

    def __init__(self, dims: S.swan_dims, P_qk: torch.Tensor, pool: PagedPool, rope_base: float = 10000.0,
                 device="cuda"):
        if dims.block_size != pool.block_size or dims.max_blocks != pool.max_blocks or \
                dims.num_blocks != pool.num_blocks or dims.B != pool.B:
            raise ValueError("dims and pool disagree on the paged geometry")
        self.pool = pool
        self._bt_version = -1
        bt = torch.from_numpy(pool.table.copy()).to(device)
        super().__init__(dims, P_qk, rope_base, device, block_table=bt)
        pool.take_dirty()  # the upload above holds every entry
        self._bt_version = pool.version

    def _to_device(self, arr, out=None):
        # pinned staging + asynchronous copy: the step does not wait for the
        # host; the caching host allocator keeps a staging buffer alive until
        # its copy has run
        staging = torch.from_numpy(np.ascontiguousarray(arr)).pin_memory()
        if out is None:
            out = torch.empty(staging.shape, dtype=staging.dtype, device=self.device)
        out.copy_(staging, non_blocking=True)
        return out

    # above this many changed entries a whole-table upload is cheaper than
    # entries carried in launch arguments (192 a launch)
    FULL_UPLOAD_ENTRIES = 4096

    def sync_table(self, copies=None, stream=None):
        """Bring the device table up to the pool's and enqueue the copy-on-write
        copies (host pairs (src, dst)).  Changed entries and copies travel in
        the arguments of swan_paged_update launches, so the step waits on no
        host-to-device copy; a table never uploaded, or with very many changes,
        is uploaded whole."""
        copies = np.zeros((0, 2), np.int32) if copies is None else np.asarray(copies, np.int32).reshape(-1, 2)
        if self._bt_version == self.pool.version and len(copies) == 0:
            return
        entries = self.pool.take_dirty()
        if self._bt_version < 0 or len(entries) > self.FULL_UPLOAD_ENTRIES:
            self._to_device(self.pool.table, self.cache.block_table)
            entries = entries[:0]
        if len(entries) or len(copies):
            S.swan_paged_update(self.dims, self.cache.struct(), self.cache.block_table, entries, copies, stream)
        self._bt_version = self.pool.version

    def _make_writable(self, pos_host):
        """Host bookkeeping of a step at positions pos_host[b]: the sparse row
        each sequence writes (-1: none) and the copy-on-write copies it needs,
        as (src, dst, row within the block)."""
        R, pool = self.dims.R, self.pool
        rows = np.asarray(pos_host, np.int64) - R
        rows = np.where(rows < 0, -1, rows)
        # most steps write into blocks the sequence already owns alone: only the
        # others (unmapped, shared, or past the table) go through prepare_write
        lb = np.where(rows >= 0, rows // pool.block_size, 0)
        blk = pool.table[np.arange(len(rows)), np.minimum(lb, pool.max_blocks - 1)]
        todo = (rows >= 0) & ((lb >= pool.max_blocks) | (blk < 0) | (pool.ref[np.maximum(blk, 0)] != 1))
        copies = []
        for b in np.flatnonzero(todo):
            cp = pool.prepare_write(int(b), int(rows[b]))
            if cp is not None:
                copies.append((cp[0], cp[1], int(rows[b]) % pool.block_size))
        return rows, copies

    def prepare_step(self, pos_host, stream=None):
        """Host side of a step at positions pos_host[b], its copies and table
        entries enqueued by swan_paged_update: returns the number of
        copy-on-write block copies."""
        _, copies = self._make_writable(pos_host)
        self.sync_table([c[:2] for c in copies], stream)
        return len(copies)

    def project_append_paged(self, q, k, v_hat, pos, pos_host, stream=None):
        """Host bookkeeping of a step, then its projection, append/evict and
        table update in one launch (swan_project_append_paged).  Takes the
        two-launch path (swan_paged_update, then swan_project_append) when
        the device table was never uploaded or has too many changes, or when
        a copy's source block is one this step appends into in place.  Returns
        the number of copy-on-write block copies."""
        rows, copies = self._make_writable(pos_host)
        pool, max_pos = self.pool, int(max(pos_host))
        w = np.flatnonzero(rows >= 0)
        lb = np.minimum(rows[w] // pool.block_size, pool.max_blocks - 1)
        appended = set(pool.table[w, lb].tolist())
        if (self._bt_version < 0 or pool.dirty_count() > self.FULL_UPLOAD_ENTRIES
                or any(c[0] in appended for c in copies)):
            self.sync_table([c[:2] for c in copies], stream)
            self.project_append(q, k, v_hat, pos, max_pos, stream)
            return len(copies)
        entries = pool.take_dirty()
        S.swan_project_append_paged(self.dims, self.cache.struct(), q, k, v_hat, pos, max_pos, self.P_qk,
                                    self.rope_base, self.q_hat, self.k_hat, self.cache.block_table, entries,
                                    np.asarray(copies, np.int32).reshape(-1, 3), stream)
        self._bt_version = pool.version
        return len(copies)

    def step_paged(self, q, k, v_hat, pos, pos_host, stream=None):
        self.project_append_paged(q, k, v_hat, pos, pos_host, stream)
        return self.decode(pos, int(max(pos_host)), stream)


def shared_prefix_pool(B: int, rows, steps: int, block_size: int, prefix_rows: int, order_fn, slack: int = 0,
                       groups: int = 1):
    """A pool for B sequences holding rows[b] sparse rows each, in `groups`
    consecutive groups of B / groups sequences (the layers of a multi-layer
    batch) whose first prefix_rows rows are the same tokens in every sequence
    of the group: the group's first sequence owns the prefix blocks and the
    others map them too (reference count B / groups); all other blocks are
    private.  Blocks come from the permutation order_fn(num_blocks) of the
    pool.  The pool has room for `steps` more rows per sequence (plus
    copy-on-write of one prefix block each) and `slack` spare blocks."""
    bs = block_size
    if groups < 1 or B % groups:
        raise ValueError("groups must divide B")
    gB = B // groups
    prefix_blocks = -(-prefix_rows // bs) if prefix_rows > 0 else 0
    have = [-(-int(r) // bs) for r in rows]
    need = [-(-(int(r) + steps) // bs) for r in rows]
    max_blocks = max(1, max(need))
    num_blocks = groups * prefix_blocks + sum(max(0, n - prefix_blocks) for n in need) + B + slack
    pool = PagedPool(num_blocks, B, max_blocks, bs, order=order_fn(num_blocks))
    for g0 in range(0, B, gB):
        for lb in range(max(have[g0], min(prefix_blocks, max_blocks))):
            pool.map_new(g0, lb)
        for b in range(g0 + 1, g0 + gB):
            pool.share(g0, b, min(prefix_blocks, have[b], have[g0]))
            for lb in range(min(prefix_blocks, have[b], have[g0]), have[b]):
                pool.map_new(b, lb)
    return pool
