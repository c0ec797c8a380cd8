"""The decode state of a synthetic workload, built on the GPU: the seeded raw
history of every sequence is generated on the host, uploaded, and converted
to the hybrid cache with swan_prefill_convert; paged workloads get a pool
whose shared-prefix blocks are mapped by every sequence of a layer.  A
multi-layer workload stacks its layers' sequences layer-major along the
batch, each layer converted in turn with its own P_QK.  The benchmark and
the full-size parity tests start from this same state."""
from __future__ import annotations

import concurrent.futures as cf
import sys
import time

import numpy as np
import torch

from . import swan as S
from . import workloads as wl
from .cache import PagedSwanDecoder, SwanDecoder, shared_prefix_pool


def _log(*a):
    print("[state]", *a, file=sys.stderr, flush=True)


def build_decoder(w: wl.Workload, split_tokens: int = 0, extra_steps: int = 0, keep_history: bool = False):
    """A SwanDecoder (PagedSwanDecoder for block_size > 0) holding workload
    w's history, with room for w.steps + extra_steps more tokens.  With
    w.layers = L > 1 the batch holds L x w.B sequences, layer l's at
    l w.B .. (l + 1) w.B - 1 (workloads.layer(w, l) drew them).  With
    keep_history (one layer only) the uploaded raw history stays on the GPU
    as dec.history = (lengths, max length, raw keys, values), the arguments
    of dec.prefill that built the cache."""
    L = max(1, w.layers)
    B, H, Bt = w.B, w.H_kv, w.B * max(1, w.layers)
    steps = w.steps + extra_steps
    T = [w.history_len(b) for b in range(B)]
    Tm = max(T)
    P = wl.projection_qk_stacked(w) if L > 1 else wl.projection_qk(w)
    P = torch.from_numpy(P).cuda()
    layers = L if L > 1 else 0
    if w.block_size > 0:
        rows = [max(0, t - w.R) for t in T] * L
        pool = shared_prefix_pool(Bt, rows, steps, w.block_size, w.shared_prefix, lambda n: wl.pool_order(w, n),
                                  w.pool_slack * L, groups=L)
        dims = S.make_dims(Bt, w.N_h, H, w.R, w.k, block_size=w.block_size, max_blocks=pool.max_blocks,
                           num_blocks=pool.num_blocks, split_tokens=split_tokens, value_format=w.value_format,
                           k_v=w.k_v, layers=layers)
        dec = PagedSwanDecoder(dims, P, pool, w.rope_base)
        _log(f"paged pool: {pool.num_blocks} blocks of {w.block_size} rows, "
             f"{int((pool.ref > 1).sum())} shared (reference count {int(pool.ref.max())})")
    else:
        dims = S.make_dims(Bt, w.N_h, H, w.R, w.k, n_cap=w.n_cap() + extra_steps + 64,
                           split_tokens=split_tokens, value_format=w.value_format, k_v=w.k_v, layers=layers)
        dec = SwanDecoder(dims, P, w.rope_base)
    K = torch.empty((B, H, Tm, 128), dtype=torch.float32, device="cuda")
    V = torch.empty_like(K)
    lens = torch.tensor(T, dtype=torch.int32, device="cuda")
    for l in range(L):
        wl_l = wl.layer(w, l) if L > 1 else w
        t0 = time.time()
        with cf.ThreadPoolExecutor(max_workers=min(16, B)) as ex:
            for b, (kb, vb) in enumerate(ex.map(lambda b: wl.history(wl_l, b), range(B))):
                K[b, :, :T[b]].copy_(torch.from_numpy(kb))
                V[b, :, :T[b]].copy_(torch.from_numpy(vb))
        if L == 1:
            _log(f"generated + uploaded history {B}x{H}x{Tm} in {time.time() - t0:.1f}s")
            dec.prefill(lens, Tm, K, V)
        else:
            # layer l alone: its sequences' planes (a paged pool: its table rows) and its P_QK
            sub = S.make_dims(B, w.N_h, H, w.R, w.k, n_cap=dims.n_cap, block_size=dims.block_size,
                              max_blocks=dims.max_blocks, num_blocks=dims.num_blocks, value_format=w.value_format,
                              k_v=w.k_v)
            S.swan_prefill_convert(sub, dec.cache.sub_struct(l * B), lens, Tm, K, V, P[l], w.rope_base)
        torch.cuda.synchronize()
    if L > 1:
        _log(f"generated, uploaded and converted {L} layers of {B}x{H}x{Tm}")
    if keep_history and L == 1:
        dec.history = (lens, Tm, K, V)
    del K, V
    torch.cuda.empty_cache()
    return dec


def step_inputs(w: wl.Workload, step: int):
    """Host inputs (q, k, v_hat, pos) of a step for the whole (stacked) batch."""
    return wl.step_inputs_stacked(w, step) if max(1, w.layers) > 1 else wl.step_inputs(w, step)
