"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split plan, state built on the GPU by
swan_prefill_convert from the seeded history).  The float64 oracle cannot
hold every sequence of these batches in reasonable time, so it runs on a
sample of sequences one by one (each sequence's state is independent of the
others); every other head is checked for a property that holds at any size:
the output is a convex combination of value vectors, so each coordinate is
bounded by the largest stored value magnitude.

Both sides build their caches from the same raw history, and the sampled
sequences' sparse rows and buffers must come out bit-exact: keys are rounded
once to fp16 from double-precision products on both sides, so the pruning
decisions agree."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_compressed_02_amd import swan as S
from decode_attention_compressed_02_amd import workloads as wl
from decode_attention_compressed_02_amd.state import build_decoder

from gpu_helpers import assert_values_bits, rel_l2_max

pytestmark = pytest.mark.gpu

TOL = 1e-3
STEPS = 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _straddling(w, dims, pos):
    """Sequences whose units share split-pass waves with the units before and
    after them: unit (b, 0) starts and unit (b, H_kv - 1) ends strictly inside a
    wave's range of work rows.  The plan is the one include/swan.h describes
    (work rows of a unit: its sparse rows plus its buffered tokens weighted by
    their bytes; V waves over equal shares of the batch)."""
    ks, ksv = S.swan_row_stride(w.k), S.swan_row_stride(w.k_v or w.k)
    row_bytes = (1 + (1 if w.value_format else 2)) * (ks + ksv)
    lens = []
    for p in pos:
        ctx = int(p) + 1
        n, f = max(ctx - w.R, 0), (0 if ctx <= 0 else min(ctx, w.R))
        lens.append(n + -(-f * 512 // row_bytes))
    H = w.H_kv
    T = H * sum(lens)
    V = min(S.swan_decode_num_splits(dims, int(max(pos))), T // 64) if dims.split_tokens == 0 else None
    assert V is not None and V >= 1
    inside = lambda x: (x * V) % T != 0  # x is not a wave boundary w T / V
    out, start = [], 0
    for b, L in enumerate(lens):
        if L and inside(start) and inside(start + H * L):
            out.append(b)
        start += H * L
    return out


def _samples(w, dims):
    """Sequences the oracle runs: the ends of the batch, a middle sequence,
    and for ragged batches the shortest, the longest and the two sequences
    nearest the middle whose units straddle waves shared with their
    neighbours (where the work plan and the merge index pieces hardest)."""
    ctx = np.asarray(w.ctx)
    if w.B <= 4:
        return sorted({1 % w.B, w.B - 1})
    if len(set(w.ctx)) == 1:
        return sorted({0, w.B // 2 - 1, w.B - 1})
    pos = wl.step_inputs(w, 0)[3]
    mid = sorted(_straddling(w, dims, pos), key=lambda b: abs(b - w.B // 2))[:2]
    assert len(mid) == 2, "a ragged batch with no straddling middle units"
    return sorted({int(np.argmax(ctx)), int(np.argmin(ctx)), w.B - 1, *mid})


def _oracle_for(w, seqs):
    sub = w.scaled(B=len(seqs), ctx=tuple(w.ctx[b] for b in seqs))
    oc = oracle.OracleCache.for_workload(sub, sub.n_cap() + STEPS)
    Tm = max(sub.history_len(i) for i in range(sub.B))
    K = np.zeros((sub.B, sub.H_kv, Tm, 128), np.float32)
    V = np.zeros_like(K)
    for i, b in enumerate(seqs):
        kb, vb = wl.history(w, b)
        K[i, :, :kb.shape[1]], V[i, :, :vb.shape[1]] = kb, vb
    oc.prefill(K, V, np.array([sub.history_len(i) for i in range(sub.B)], np.int64),
               wl.projection_qk(w).astype(np.float64), w.rope_base, oracle.default_threads())
    return oc


def _seq_rows(dec, b, n):
    """GPU sparse planes of sequence b, rows [0, n): 4 arrays [H][n][k_stride]."""
    d, planes = dec.dims, dec.cache.sparse_views()
    if d.block_size == 0:
        return [p[b, :, :n].cpu().numpy() for p in planes]
    bs = d.block_size
    blk = torch.from_numpy(dec.pool.table[b, :-(-n // bs)].astype(np.int64)).cuda()
    out = []
    for p in planes:  # [num_blocks][H][bs][ks] -> [H][rows][ks]
        g = p.index_select(0, blk).permute(1, 0, 2, 3).reshape(d.H_kv, -1, p.shape[-1])
        out.append(g[:, :n].cpu().numpy())
    return out


def _check_rows(dec, oc, seqs, w, lo, ns):
    """Rows [lo, ns[i]) of the sampled sequences, and their dense buffers,
    bit-exact against the oracle."""
    for i, b in enumerate(seqs):
        n = ns[i]
        if n <= lo:
            continue
        ki, kv, vi, vv = _seq_rows(dec, b, n)
        k_v = w.k_v or w.k  # kept value coordinates
        np.testing.assert_array_equal(ki[:, lo:n, :w.k], oc.kidx[i, :, lo:n])
        np.testing.assert_array_equal(vi[:, lo:n, :k_v], oc.vidx[i, :, lo:n])
        assert_values_bits(kv[:, lo:n, :w.k], oc.kval[i, :, lo:n], w.value_format)
        assert_values_bits(vv[:, lo:n, :k_v], oc.vval[i, :, lo:n], w.value_format)
    if w.R > 0:
        kb, vb = dec.cache.buffer_views()
        for i, b in enumerate(seqs):
            np.testing.assert_array_equal(kb[b].cpu().numpy().astype(np.float64), oc.ringk[i])
            np.testing.assert_array_equal(vb[b].cpu().numpy().astype(np.float64), oc.ringv[i])


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, "3-fp8", "5-fp8", "2-kv"])
def test_full_size_steps(cfg):
    w = wl.config(int(str(cfg)[0]))
    if str(cfg).endswith("fp8"):  # the same workload with 8-bit sparse values
        w = w.scaled(value_format=1)
    if str(cfg).endswith("kv"):  # its 2k budget split 60/40 between keys and values (77 / 51)
        w = w.scaled(k=77, k_v=51)
    print(f"\n[fullsize] workload {cfg}: {w.name} B={w.B}", flush=True)
    dec = build_decoder(w, extra_steps=STEPS)
    seqs = _samples(w, dec.dims)
    print(f"[fullsize] samples {seqs}", flush=True)
    print(f"[fullsize] GPU state built; split waves "
          f"{S.swan_decode_num_splits(dec.dims, int(max(w.ctx)) + STEPS)}", flush=True)
    oc = _oracle_for(w, seqs)
    print("[fullsize] oracle state built", flush=True)
    n0 = [max(0, w.history_len(b) - w.R) for b in seqs]
    _check_rows(dec, oc, seqs, w, 0, n0)
    print("[fullsize] prefilled rows and buffers of the samples are bit-exact", flush=True)
    P64 = wl.projection_qk(w).astype(np.float64)
    for s in range(STEPS):
        q, kr, vn, pos = wl.step_inputs(w, s)
        cu = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q, kr, vn, pos)]
        if w.block_size > 0:  # the benchmark's paged step: table update, projection and append in one launch
            out = dec.step_paged(*cu, pos)
        else:
            out = dec.step(*cu, int(pos.max()))
        _, _, want = oc.step(q[seqs], kr[seqs], vn[seqs], pos[seqs].astype(np.int64), P64, w.rope_base,
                             oracle.default_threads())
        got = out[seqs].cpu().numpy()
        err = rel_l2_max(got, want)
        # every head: finite and bounded by the largest stored value
        vmax = float(dec.cache.v_buf.abs().max())
        if w.value_format:  # E4M3 bytes: the largest magnitude code of the plane
            vmax = max(vmax, float(dec.cache.v_val.view(torch.float8_e4m3fn).float().abs().max()))
        else:
            vmax = max(vmax, float(dec.cache.v_val.abs().max()))
        bound = float(out.abs().max())
        print(f"[fullsize] workload {cfg} step {s}: sampled rel_l2={err:.2e}; max|o|={bound:.3f} <= {vmax:.3f}",
              flush=True)
        assert torch.isfinite(out).all()
        assert bound <= vmax * (1 + 1e-5)
        assert err < TOL
    # rows the steps appended (tokens evicted from the buffer)
    _check_rows(dec, oc, seqs, w, min(n0), [w.n_after(b, STEPS - 1) for b in seqs])
