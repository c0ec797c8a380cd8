"""Seeded synthetic inputs for the SWAN hybrid-cache decode step.

This module only *draws* inputs: raw (pre-RoPE) queries and keys, the values a
model with the absorbed value projection emits, random orthogonal projection
matrices, context lengths and the physical-block order of a paged pool.  It
contains none of the method's arithmetic (no RoPE, no projection, no pruning,
no attention), so the HIP path and the CPU oracle can both consume it without
sharing any step of the computation.

Workloads follow the head layout the SWAN page evaluates on (Llama-3.1-8B:
32 query heads, 8 kv heads, d_h = 128; SWAN page, GSM8K and NLP-benchmark
sections) and the dense-buffer sizes it uses (64 and 128 tokens, plus 256 for
the long batch).  All randomness comes from numpy's PCG64 seeded per
(workload seed, stream, sequence) so any single sequence can be regenerated
on its own.

Conventions shared by both consumers (stated here because they are input
conventions, not arithmetic):

* ``ctx[b]`` is the number of tokens sequence ``b`` attends to at its first
  decode step, the new token included.  The new token of step ``s`` sits at
  position ``ctx[b] - 1 + s``; the prefilled history is positions
  ``0 .. ctx[b] - 2``.
* Raw keys are drawn pre-RoPE (RoPE and P_QK are applied at run time, SWAN
  page, projection section).  Values are drawn in the basis the cache stores
  them in: a model whose value weights absorbed P_VO emits rotated values
  directly (SWAN page, absorption paragraph), so there is nothing for the
  decode step to rotate.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

D_H = 128

# stream ids for the per-purpose generators
_S_PROJ, _S_VO, _S_OUTLIER, _S_DRIFT, _S_HIST, _S_PREFIX, _S_STEP, _S_LEN, _S_POOL = range(9)


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic decode workload."""

    name: str
    B: int
    N_h: int
    H_kv: int
    R: int
    k: int
    ctx: tuple  # tokens attended at the first step, per sequence
    steps: int = 1
    d_h: int = D_H
    seed: int = 0
    rope_base: float = 10000.0
    outlier_channels: int = 0  # per kv-head, in K (raw basis) and V (stored basis)
    outlier_scale: float = 1.0
    drift_amp: float = 0.0  # per-channel sinusoidal mean drift of raw keys
    drift_period: tuple = (256.0, 65536.0)
    block_size: int = 0  # 0: contiguous sparse rows; >0: paged blocks of this many rows
    shared_prefix: int = 0  # tokens whose K/V are identical across all sequences
    pool_slack: int = 0  # extra free blocks in the paged pool
    value_format: int = 0  # sparse values: 0 fp16, 1 fp8 E4M3 (storage only; the inputs are the same)
    k_v: int = 0  # value coordinates kept, 0 = k (keys and values keeping different shares)
    layers: int = 1  # layers stacked along the batch (each B sequences; see layer())

    @property
    def g(self) -> int:
        return self.N_h // self.H_kv

    def pos0(self) -> np.ndarray:
        """Position of the new token at step 0, per sequence."""
        return np.asarray(self.ctx, dtype=np.int64) - 1

    def history_len(self, b: int) -> int:
        return int(self.ctx[b]) - 1

    def n_after(self, b: int, step: int) -> int:
        """Sparse rows of sequence b after step ``step`` appended its token."""
        return max(0, int(self.ctx[b]) + step - self.R)

    def n_cap(self) -> int:
        """Sparse rows needed per sequence to run all steps."""
        return max(self.n_after(b, self.steps - 1) for b in range(self.B))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _rng(w: Workload, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([int(w.seed), stream, *[int(e) for e in extra]])


def random_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed orthogonal d x d matrix: QR of a Gaussian with the
    signs of R's diagonal folded into Q (float64)."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q *= np.sign(np.diag(r))[None, :]
    return q


def projection_qk(w: Workload) -> np.ndarray:
    """P_QK per kv-head, float32 [H_kv][d_h][d_h], row-vector convention x·P.

    One independent random orthogonal matrix per kv-head stands in for the
    learned per-head bases (the SWAN page's projection ablation also uses a
    random orthogonal basis)."""
    rng = _rng(w, _S_PROJ)
    return np.stack([random_orthogonal(rng, w.d_h) for _ in range(w.H_kv)]).astype(np.float32)


def projection_vo(w: Workload) -> np.ndarray:
    """P_VO per kv-head (float64), used only where a test un-rotates outputs."""
    rng = _rng(w, _S_VO)
    return np.stack([random_orthogonal(rng, w.d_h) for _ in range(w.H_kv)])


def _outlier_sets(w: Workload):
    """(K channels, V channels) per kv-head scaled by ``outlier_scale``."""
    if w.outlier_channels <= 0:
        return None
    rng = _rng(w, _S_OUTLIER)
    kc = [np.sort(rng.choice(w.d_h, w.outlier_channels, replace=False)) for _ in range(w.H_kv)]
    vc = [np.sort(rng.choice(w.d_h, w.outlier_channels, replace=False)) for _ in range(w.H_kv)]
    return kc, vc


def _drift_params(w: Workload):
    """Per (kv-head, channel) period T_c (log-uniform) and phase phi_c."""
    rng = _rng(w, _S_DRIFT)
    lo, hi = np.log(w.drift_period[0]), np.log(w.drift_period[1])
    period = np.exp(rng.uniform(lo, hi, size=(w.H_kv, w.d_h)))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(w.H_kv, w.d_h))
    return period, phase


def _shape_keys(w: Workload, K: np.ndarray, positions: np.ndarray) -> None:
    """Apply the workload's outlier scaling and positional drift to raw keys
    K [H_kv][T][d] in place (input synthesis, before any RoPE)."""
    sets = _outlier_sets(w)
    if sets is not None:
        for h in range(w.H_kv):
            K[h][:, sets[0][h]] *= w.outlier_scale
    if w.drift_amp != 0.0:
        period, phase = _drift_params(w)
        t = positions.astype(np.float64)[None, :, None]
        K += (w.drift_amp * np.sin(2.0 * np.pi * t / period[:, None, :] + phase[:, None, :])).astype(K.dtype)


def _shape_values(w: Workload, V: np.ndarray) -> None:
    sets = _outlier_sets(w)
    if sets is not None:
        for h in range(w.H_kv):
            V[h][:, sets[1][h]] *= w.outlier_scale


def _draw_kv(rng: np.random.Generator, H: int, T: int, d: int):
    K = rng.standard_normal((H, T, d), dtype=np.float32)
    V = rng.standard_normal((H, T, d), dtype=np.float32)
    return K, V


def history(w: Workload, b: int, t0: int = 0, t1: int | None = None):
    """Raw keys and stored-basis values of the prefilled history of sequence
    ``b``: float32 arrays [H_kv][T][d_h] for positions ``t0 .. t1-1``
    (default: the whole history ``0 .. ctx[b]-2``).

    With ``shared_prefix`` > 0, positions below it are the same for every
    sequence (a shared system prompt).  Blocks of 4096 positions are drawn
    from their own streams so any window can be regenerated cheaply."""
    T = w.history_len(b)
    t1 = T if t1 is None else min(t1, T)
    out_k = np.empty((w.H_kv, max(0, t1 - t0), w.d_h), np.float32)
    out_v = np.empty_like(out_k)
    blk = 4096
    t = t0
    while t < t1:
        c = t // blk
        lo, hi = c * blk, (c + 1) * blk
        if hi <= w.shared_prefix:
            rng = _rng(w, _S_PREFIX, c)
        elif lo >= w.shared_prefix:
            rng = _rng(w, _S_HIST, b, c)
        else:  # block straddles the prefix end: draw both and splice
            rng = None
        if rng is not None:
            K, V = _draw_kv(rng, w.H_kv, blk, w.d_h)
        else:
            Kp, Vp = _draw_kv(_rng(w, _S_PREFIX, c), w.H_kv, blk, w.d_h)
            Ks, Vs = _draw_kv(_rng(w, _S_HIST, b, c), w.H_kv, blk, w.d_h)
            cut = w.shared_prefix - lo
            K = np.concatenate([Kp[:, :cut], Ks[:, cut:]], axis=1)
            V = np.concatenate([Vp[:, :cut], Vs[:, cut:]], axis=1)
        a, e = t - lo, min(t1, hi) - lo
        out_k[:, t - t0:t - t0 + (e - a)] = K[:, a:e]
        out_v[:, t - t0:t - t0 + (e - a)] = V[:, a:e]
        t = lo + e
    _shape_keys(w, out_k, np.arange(t0, t1))
    _shape_values(w, out_v)
    return out_k, out_v


def step_inputs(w: Workload, step: int):
    """Inputs of decode step ``step``: raw queries float32 [B][N_h][d_h], raw
    new keys float32 [B][H_kv][d_h], new stored-basis values float32
    [B][H_kv][d_h], and positions int32 [B]."""
    rng = _rng(w, _S_STEP, step)
    q = rng.standard_normal((w.B, w.N_h, w.d_h), dtype=np.float32)
    k = rng.standard_normal((w.B, w.H_kv, w.d_h), dtype=np.float32)
    v = rng.standard_normal((w.B, w.H_kv, w.d_h), dtype=np.float32)
    pos = (w.pos0() + step).astype(np.int32)
    for b in range(w.B):
        kb = k[b][:, None, :].copy()
        _shape_keys(w, kb, np.array([pos[b]]))
        k[b] = kb[:, 0, :]
        vb = v[b][:, None, :].copy()
        _shape_values(w, vb)
        v[b] = vb[:, 0, :]
    return q, k, v, pos


# ---------------------------------------------------------------------------
# Several layers in one batch: the library stacks the sequences of all layers
# layer-major along its batch.  Layer l of a workload has the same shapes and
# context lengths and its own inputs, drawn from seed + _LAYER_SEED_STRIDE l.
# ---------------------------------------------------------------------------

_LAYER_SEED_STRIDE = 7919


def layer(w: Workload, l: int) -> Workload:
    """Layer ``l`` (0-based) of a multi-layer workload, as a one-layer workload."""
    return w.scaled(seed=w.seed + _LAYER_SEED_STRIDE * l, layers=1)


def projection_qk_stacked(w: Workload) -> np.ndarray:
    """P_QK of every layer, float32 [layers][H_kv][d_h][d_h] (a layer is
    [H_kv][d_h][d_h], as projection_qk gives it)."""
    return np.stack([projection_qk(layer(w, l)) for l in range(max(1, w.layers))])


def step_inputs_stacked(w: Workload, step: int):
    """step_inputs of every layer, concatenated layer-major along the batch."""
    parts = [step_inputs(layer(w, l), step) for l in range(max(1, w.layers))]
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def pool_order(w: Workload, num_blocks: int) -> np.ndarray:
    """Order in which a paged pool hands out its physical blocks: a random
    permutation of ``0 .. num_blocks-1`` (int32)."""
    return _rng(w, _S_POOL).permutation(num_blocks).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds are 1000 + workload number.
# ---------------------------------------------------------------------------

def _ragged_ctx(seed: int, n: int, lo: int, hi: int) -> tuple:
    rng = np.random.default_rng([seed, _S_LEN])
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


def config(i: int) -> Workload:
    """Workload ``i`` (1..5):

    1. one sequence, one head, n = 2048 sparse + R = 128, k = 32;
    2. Llama-3-8B layer, batch 8, context 8192, R = 128, k = 64, four
       outlier channels x8 per kv-head in K and V;
    3. batch 16, context 32768, R = 256, k = 32, 16 consecutive steps;
    4. batch 4, context 131072, R = 128, k = 32, keys with a per-channel
       sinusoidal mean drift of amplitude 0.5;
    5. 32 ragged sequences (context uniform in [1024, 16384]), R = 64,
       k = 64, 16-row paged blocks, a shared 1536-token prefix.
    """
    seed = 1000 + i
    if i == 1:
        return Workload("single-seq n2048 R128 k32", 1, 1, 1, 128, 32, (2176,), seed=seed)
    if i == 2:
        return Workload("gqa b8 ctx8192 R128 k64 outliers", 8, 32, 8, 128, 64, (8192,) * 8, seed=seed,
                        outlier_channels=4, outlier_scale=8.0)
    if i == 3:
        return Workload("gqa b16 ctx32768 R256 k32 16 steps", 16, 32, 8, 256, 32, (32768,) * 16, steps=16,
                        seed=seed)
    if i == 4:
        return Workload("gqa b4 ctx131072 R128 k32 drift", 4, 32, 8, 128, 32, (131072,) * 4, seed=seed,
                        drift_amp=0.5)
    if i == 5:
        return Workload("paged ragged b32 ctx1024-16384 R64 k64", 32, 32, 8, 64, 64,
                        _ragged_ctx(seed, 32, 1024, 16384), seed=seed, block_size=16, shared_prefix=1536,
                        pool_slack=64)
    raise ValueError(f"no workload {i}")
