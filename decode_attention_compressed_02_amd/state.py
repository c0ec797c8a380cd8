"""The decode state of a synthetic workload, built on the GPU: the seeded raw
history of every sequence is generated on the host, uploaded, and converted
to the hybrid cache with swan_prefill_convert; paged workloads get a pool
whose shared-prefix blocks are mapped by every sequence.  The benchmark and
the full-size parity tests start from this same state."""
from __future__ import annotations

import concurrent.futures as cf
import sys
import time

import torch

from . import swan as S
from . import workloads as wl
from .cache import PagedSwanDecoder, SwanDecoder, shared_prefix_pool


def _log(*a):
    print("[state]", *a, file=sys.stderr, flush=True)


def build_decoder(w: wl.Workload, split_tokens: int = 0, extra_steps: int = 0):
    """A SwanDecoder (PagedSwanDecoder for block_size > 0) holding workload
    w's history, with room for w.steps + extra_steps more tokens."""
    B, H = w.B, w.H_kv
    steps = w.steps + extra_steps
    T = [w.history_len(b) for b in range(B)]
    Tm = max(T)
    P = torch.from_numpy(wl.projection_qk(w)).cuda()
    if w.block_size > 0:
        rows = [max(0, t - w.R) for t in T]
        pool = shared_prefix_pool(B, rows, steps, w.block_size, w.shared_prefix, lambda n: wl.pool_order(w, n),
                                  w.pool_slack)
        dims = S.make_dims(w.B, w.N_h, w.H_kv, w.R, w.k, block_size=w.block_size, max_blocks=pool.max_blocks,
                           num_blocks=pool.num_blocks, split_tokens=split_tokens, value_format=w.value_format,
                           k_v=w.k_v)
        dec = PagedSwanDecoder(dims, P, pool, w.rope_base)
        _log(f"paged pool: {pool.num_blocks} blocks of {w.block_size} rows, "
             f"{int((pool.ref > 1).sum())} shared (reference count {int(pool.ref.max())})")
    else:
        dims = S.make_dims(w.B, w.N_h, w.H_kv, w.R, w.k, n_cap=w.n_cap() + extra_steps + 64,
                           split_tokens=split_tokens, value_format=w.value_format, k_v=w.k_v)
        dec = SwanDecoder(dims, P, w.rope_base)
    K = torch.empty((B, H, Tm, 128), dtype=torch.float32, device="cuda")
    V = torch.empty_like(K)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=min(16, B)) as ex:
        for b, (kb, vb) in enumerate(ex.map(lambda b: wl.history(w, b), range(B))):
            K[b, :, :T[b]].copy_(torch.from_numpy(kb))
            V[b, :, :T[b]].copy_(torch.from_numpy(vb))
    _log(f"generated + uploaded history {B}x{H}x{Tm} in {time.time() - t0:.1f}s")
    lens = torch.tensor(T, dtype=torch.int32, device="cuda")
    dec.prefill(lens, Tm, K, V)
    torch.cuda.synchronize()
    del K, V
    torch.cuda.empty_cache()
    return dec
