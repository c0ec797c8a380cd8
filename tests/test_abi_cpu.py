"""The C-ABI library without a GPU: it loads, exports every entry point
include/swan.h declares, sizes its buffers, and rejects bad arguments with
the documented status before enqueuing anything."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from decode_attention_compressed_02_amd import swan as S  # noqa: E402


def declared_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", h)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(swan_[a-z0-9_]+)\s*\(", txt))
    return sorted(names)


def test_header_and_binding_agree():
    assert declared_functions() == sorted(S.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = C.CDLL(S.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), f"{name} not exported as text symbol"


def test_row_stride_and_sizes():
    assert [S.swan_row_stride(k) for k in (1, 7, 8, 9, 16, 24, 32, 33, 64, 100, 128)] == \
        [8, 8, 8, 16, 16, 32, 32, 64, 64, 128, 128]
    d = S.make_dims(16, 32, 8, 256, 32, n_cap=32528)
    n_idx, n_val, nv_idx, nv_val, n_buf = S.swan_cache_bytes(d)
    assert n_idx == 16 * 8 * 32528 * 32 and n_val == 2 * n_idx and (nv_idx, nv_val) == (n_idx, n_val)
    assert n_buf == 16 * 8 * 256 * 128 * 2
    dp = S.make_dims(32, 32, 8, 64, 64, block_size=16, max_blocks=1024, num_blocks=20000)
    assert S.swan_cache_bytes(dp)[0] == 20000 * 8 * 16 * 64
    # 8-bit values: one byte per value entry, the dense buffer stays fp16
    d8 = S.make_dims(16, 32, 8, 256, 32, n_cap=32528, value_format=S.SWAN_VALUES_FP8_E4M3)
    assert S.swan_cache_bytes(d8) == (n_idx, n_idx, n_idx, n_idx, n_buf)
    # keys keep 77 (stride 128), values 51 (stride 64)
    da = S.make_dims(2, 8, 2, 16, 77, n_cap=100, k_v=51)
    rows = 2 * 2 * 100
    assert S.swan_cache_bytes(da) == (rows * 128, rows * 256, rows * 64, rows * 128, 2 * 2 * 16 * 128 * 2)


def test_size_limits():
    # the largest contiguous unit a 32-bit buffer range covers: 2^24 - 1 rows of 128 fp16 entries
    assert S.swan_cache_bytes(S.make_dims(1, 4, 1, 0, 128, n_cap=(1 << 24) - 1))[1] == ((1 << 24) - 1) * 256
    # paged row slots are 64-bit: a pool of more than 2^31 rows (of 8-entry rows) is accepted
    d = S.make_dims(4, 8, 8, 64, 8, block_size=16, max_blocks=1 << 20, num_blocks=1 << 24)
    assert S.swan_cache_bytes(d)[0] == (1 << 24) * 8 * 16 * 8


def test_split_plan():
    d = S.make_dims(16, 32, 8, 256, 32, n_cap=40000)
    # first step of the batch-16 32K workload: per (sequence, kv head) 32512
    # sparse rows + 256 buffered tokens of 256 / 96 work rows each (683 in
    # all) = 33195 work rows; 128 units.  One wave per resident slot (the
    # split kernel's 34 KB of LDS fits 4 per CU; 256 CUs) -> 1024 waves.
    W = S.swan_decode_num_splits(d, 32767)
    assert W == 1024
    # partials: at most W + B H_kv pieces, g = 4 heads each, 128 + 2 floats
    assert S.swan_decode_workspace_bytes(d, 32767) == (1024 + 128) * 4 * 130 * 4
    d.split_tokens = 1024
    assert S.swan_decode_num_splits(d, 32767) == _ceil(128 * 33195, 1024)  # 4150
    d.R = 0
    assert S.swan_decode_num_splits(d, 32767) == 128 * 32768 // 1024
    assert S.swan_decode_num_splits(S.make_dims(1, 1, 1, 128, 32, n_cap=0), -1) == 1
    # only buffered tokens (context 200 <= R): ceil(200 * 256 / 96) = 534
    # work rows per unit, 4 units, at least 64 rows per wave -> 33 waves
    assert S.swan_decode_num_splits(S.make_dims(2, 8, 2, 256, 32, n_cap=10), 199) == 33
    d2 = S.make_dims(1, 1, 1, 0, 32, n_cap=1 << 20, split_tokens=64)
    assert S.swan_decode_num_splits(d2, (1 << 20) - 1) == (1 << 20) // 64


def _ceil(a, b):
    return -(-a // b)


def _unit(p, R, ks, row_cap):
    ctx = p + 1
    n = min(max(ctx - R, 0), row_cap)
    f = 0 if ctx <= 0 else min(ctx, R)
    return n, f, n + _ceil(f * 256, 3 * ks)


def _active_waves(T, W, st):
    v = _ceil(T, st) if st > 0 else T // 64
    return max(1, min(v, W))


def _plan_pieces(pos, H, W, split_tokens, R, ks, row_cap):
    """The split pass's work plan written out on the host: for every wave,
    its pieces (b, h, sparse rows [t0, t1), buffered tokens [d0, d1), partial
    index).  It follows the kernel's integer arithmetic so that the plan's
    invariants can be checked here; the GPU parity tests check the kernel."""
    def sparse_split(x, n, L):
        return n if x >= L else min(x * _ceil(n, 16) // L * 16, n)

    def dense_split(x, f, L):
        return f if x >= L else _ceil(x * f, L)

    units = [_unit(p, R, ks, row_cap) for p in pos]
    T = H * sum(u[2] for u in units)
    V = _active_waves(T, W, split_tokens)
    pieces = []
    for w in range(V):
        x0, x1 = w * T // V, (w + 1) * T // V
        P = 0
        for b, (n, f, L) in enumerate(units):
            for h in range(H):
                us = P + h * L
                lo, hi = max(x0, us) - us, min(x1, us + L) - us
                if L == 0 or lo >= hi:
                    continue
                pieces.append((w, b, h, sparse_split(lo, n, L), sparse_split(hi, n, L),
                               dense_split(lo, f, L), dense_split(hi, f, L), w + b * H + h))
            P += H * L
    return units, pieces, T, V


@pytest.mark.parametrize("pos,H,W,st,R,ks", [
    ([1023, 16383, 5000, 64, -1, 300], 8, 1024, 0, 64, 64),
    ([32767] * 4, 8, 1024, 0, 256, 32),
    ([32767] * 16, 8, 1024, 0, 256, 32),
    ([130, 17, 2000, 99999], 2, 37, 0, 128, 16),
    ([4000, 1, 0, 70000], 3, 1 << 20, 128, 128, 128),
])
def test_work_plan_partitions_every_unit(pos, H, W, st, R, ks):
    units, pieces, T, V = _plan_pieces(pos, H, W, st, R, ks, 1 << 20)
    # every sparse row and buffered token of every unit lies in exactly one piece
    for b, (n, f, L) in enumerate(units):
        for h in range(H):
            mine = [p for p in pieces if p[1] == b and p[2] == h]
            rows = sorted(r for p in mine for r in range(p[3], max(p[3], p[4])))
            toks = sorted(t for p in mine for t in range(p[5], max(p[5], p[6])))
            assert rows == list(range(n)) and toks == list(range(f))
            # a ring slot never straddles a 16-row block
            assert all(p[3] % 16 == 0 or p[3] == p[4] for p in mine)
            # equal pieces carry the unit's mix of sparse rows and buffered tokens
            if len(mine) > 2 and f > 0:
                inner = mine[1:-1]
                assert max(p[6] - p[5] for p in inner) - min(p[6] - p[5] for p in inner) <= 1
    idx = [p[7] for p in pieces]
    assert len(set(idx)) == len(idx) and max(idx, default=0) < V + len(pos) * H
    # equal units and a wave count that is a multiple of the unit count: one piece per wave
    if len(set(pos)) == 1 and V % (len(pos) * H) == 0:
        assert len(pieces) == V
    # the reduce finds a unit's pieces as the waves ceil((us + 1) V / T) - 1 ..
    # ceil((us + L) V / T) - 1
    P = 0
    for b, (n, f, L) in enumerate(units):
        for h in range(H):
            us = P + h * L
            waves = sorted(p[0] for p in pieces if p[1] == b and p[2] == h)
            w0, w1 = max(_ceil((us + 1) * V, T) - 1, 0), min(_ceil((us + L) * V, T) - 1, V - 1)
            assert waves == (list(range(w0, w1 + 1)) if L else [])
        P += H * L


ERROR_CASES = r'''
import ctypes as C, sys
sys.path.insert(0, ROOT)
from decode_attention_compressed_02_amd import swan as S
L = S.lib()
F = C.c_void_p(0x1000)  # never dereferenced: every case below must fail validation
N = None
def dims(**kw):
    d = S.make_dims(2, 8, 2, 16, 32, n_cap=100)
    for k, v in kw.items(): setattr(d, k, v)
    return d
cache = S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None)
nocache = S.swan_cache(0x1000, 0x1000, None, 0x1000, 0x1000, 0x1000, None)
st = C.c_void_p(0)
def proj(d, **kw):
    a = dict(q=F, k=F, pos=F, P=F, base=10000.0, qh=F, kh=F); a.update(kw)
    return L.swan_project_qk(C.byref(d), a['q'], a['k'], a['pos'], a['P'], a['base'], a['qh'], a['kh'], st)
def app(d, c=cache, max_pos=50, **kw):
    a = dict(pos=F, kh=F, vh=F); a.update(kw)
    return L.swan_append_evict(C.byref(d), C.byref(c), a['pos'], max_pos, a['kh'], a['vh'], st)
def dec(d, c=cache, max_pos=50, ws_bytes=1 << 30, **kw):
    a = dict(pos=F, qh=F, oh=F, ws=F); a.update(kw)
    return L.swan_decode_attn(C.byref(d), C.byref(c), a['pos'], max_pos, a['qh'], a['oh'], a['ws'], ws_bytes, st)
def pa(d, c=cache, max_pos=50, **kw):
    a = dict(q=F, k=F, vh=F, pos=F, P=F, base=10000.0, qh=F, kh=F); a.update(kw)
    return L.swan_project_append(C.byref(d), C.byref(c), a['q'], a['k'], a['vh'], a['pos'], max_pos, a['P'],
                                 a['base'], a['qh'], a['kh'], st)
pcache = S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x2000)
pdims = lambda: dims(block_size=16, max_blocks=4, num_blocks=8)  # B 2: table slots 0..7
def pairs(*xs):
    return (C.c_int32 * max(1, len(xs)))(*xs)
def upd(d, c=pcache, table=0x2000, entries=pairs(0, 3), ne=1, copies=pairs(1, 2), nc=1):
    return L.swan_paged_update(C.byref(d), C.byref(c), C.c_void_p(table) if table else None, entries, ne, copies, nc, st)
def pap(d, c=pcache, table=0x2000, entries=pairs(0, 3), ne=1, copies=pairs(1, 2, 0), nc=1, max_pos=50, **kw):
    a = dict(q=F, k=F, vh=F, pos=F, P=F, base=10000.0, qh=F, kh=F); a.update(kw)
    return L.swan_project_append_paged(C.byref(d), C.byref(c), a['q'], a['k'], a['vh'], a['pos'], max_pos, a['P'],
                                       a['base'], a['qh'], a['kh'], C.c_void_p(table) if table else None, entries, ne,
                                       copies, nc, st)
def pre(d, c=cache, max_len=40, T=64, **kw):
    a = dict(len=F, kr=F, vh=F, P=F); a.update(kw)
    return L.swan_prefill_convert(C.byref(d), C.byref(c), a['len'], max_len, T, a['kr'], a['vh'], a['P'], 10000.0, st)
E, U, CAP = S.SWAN_ERR_INVALID_ARG, S.SWAN_ERR_UNSUPPORTED, S.SWAN_ERR_CAPACITY
cases = [
    ("d_h 64", proj(dims(d_h=64)), U),
    ("g = 3", proj(dims(N_h=6, H_kv=2)), U),
    ("g = 16", proj(dims(N_h=32, H_kv=2)), U),
    ("N_h % H_kv", proj(dims(N_h=7, H_kv=2)), E),
    ("k = 0", proj(dims(k=0)), E),
    ("k > d_h", proj(dims(k=129)), E),
    ("R < 0", proj(dims(R=-1)), E),
    ("B = 0", proj(dims(B=0)), E),
    ("split_tokens not /64", dec(dims(split_tokens=100)), E),
    ("value format 2", proj(dims(value_format=2)), U),
    ("k_v > d_h", proj(dims(k_v=129)), E),
    ("k_v < 0", proj(dims(k_v=-1)), E),
    ("k_v stride 4x k's", dec(dims(k=8, k_v=32)), U),
    ("k_v stride 8x k's", app(dims(k=128, k_v=16)), U),
    ("value format -1", dec(dims(value_format=-1)), U),
    ("layers not dividing B", proj(dims(layers=3)), E),
    ("layers < 0", dec(dims(layers=-1)), E),
    ("null q", proj(dims(), q=N), E),
    ("null k_hat out", proj(dims(), kh=N), E),
    ("rope base 1", proj(dims(), base=1.0), E),
    ("null dims", L.swan_project_qk(None, F, F, F, F, 10000.0, F, F, st), E),
    ("append null plane", app(dims(), c=nocache), E),
    ("append null pos", app(dims(), pos=N), E),
    ("append capacity", app(dims(), max_pos=100 + 16), CAP),
    ("append capacity R=0", app(dims(R=0), max_pos=100), CAP),
    ("paged without table", app(dims(block_size=16, max_blocks=4, num_blocks=8)), E),
    ("paged capacity", app(dims(block_size=16, max_blocks=4, num_blocks=8),
                           c=S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000), max_pos=16 * 4 + 16), CAP),
    ("decode capacity", dec(dims(), max_pos=100 + 16), CAP),
    ("decode workspace small", dec(dims(), ws_bytes=16), E),
    ("decode null workspace", dec(dims(), ws=N), E),
    ("decode null q_hat", dec(dims(), qh=N), E),
    ("decode null pos", dec(dims(), pos=N), E),
    ("decode too many waves", dec(dims(split_tokens=64, n_cap=1 << 25), max_pos=(1 << 25) - 1), E),
    ("project+append null v_hat", pa(dims(), vh=N), E),
    ("project+append null plane", pa(dims(), c=nocache), E),
    ("project+append capacity", pa(dims(), max_pos=100 + 16), CAP),
    ("project+append rope base", pa(dims(), base=0.5), E),
    ("project+append g = 3", pa(dims(N_h=6, H_kv=2)), U),
    ("prefill capacity", pre(dims(), max_len=100 + 17, T=200), CAP),
    ("prefill T_stride < max_len", pre(dims(), max_len=70, T=64), E),
    ("prefill null raw keys", pre(dims(), kr=N), E),
    ("copy blocks contiguous", L.swan_copy_blocks(C.byref(dims()), C.byref(cache), F, F, 1, st), E),
    ("copy blocks count < 0", L.swan_copy_blocks(C.byref(dims(block_size=16, max_blocks=4, num_blocks=8)),
                                                 C.byref(S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)),
                                                 F, F, -1, st), E),
    ("copy blocks null ids", L.swan_copy_blocks(C.byref(dims(block_size=16, max_blocks=4, num_blocks=8)),
                                                C.byref(S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)),
                                                N, F, 2, st), E),
    ("copy blocks odd block bytes", L.swan_copy_blocks(C.byref(dims(H_kv=1, N_h=1, k=8, block_size=1, max_blocks=4, num_blocks=8)),
                                                       C.byref(S.swan_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)),
                                                       F, F, 1, st), U),
]
cases += [
    ("paged update contiguous", upd(dims(), c=cache), E),
    ("paged update other table", upd(pdims(), table=0x3000), E),
    ("paged update null table", upd(pdims(), table=0), E),
    ("paged update slot past the table", upd(pdims(), entries=pairs(8, 3)), E),
    ("paged update negative slot", upd(pdims(), entries=pairs(-1, 3)), E),
    ("paged update block past the pool", upd(pdims(), entries=pairs(0, 8)), E),
    ("paged update block -2", upd(pdims(), entries=pairs(0, -2)), E),
    ("paged update copy onto itself", upd(pdims(), copies=pairs(2, 2)), E),
    ("paged update copy past the pool", upd(pdims(), copies=pairs(1, 9)), E),
    ("paged update negative count", upd(pdims(), ne=-1), E),
    ("paged update null entries", upd(pdims(), entries=None, ne=2), E),
    ("paged update null copies", upd(pdims(), copies=None, nc=1), E),
    ("paged update odd block bytes", upd(dims(H_kv=1, N_h=1, k=8, block_size=1, max_blocks=4, num_blocks=8)), U),
    ("paged step contiguous", pap(dims(), c=cache), E),
    ("paged step other table", pap(pdims(), table=0x3000), E),
    ("paged step repeated slot", pap(pdims(), entries=pairs(0, 3, 0, 4), ne=2), E),
    ("paged step slot past the table", pap(pdims(), entries=pairs(8, 3)), E),
    ("paged step skip row past the block", pap(pdims(), copies=pairs(1, 2, 16)), E),
    ("paged step skip row -2", pap(pdims(), copies=pairs(1, 2, -2)), E),
    ("paged step copy onto itself", pap(pdims(), copies=pairs(2, 2, 0)), E),
    ("paged step negative count", pap(pdims(), nc=-1), E),
    ("paged step null copies", pap(pdims(), copies=None, nc=1), E),
    ("paged step null v_hat", pap(pdims(), vh=N), E),
    ("paged step capacity", pap(pdims(), max_pos=16 * 4 + 16), CAP),
    ("paged step g = 3", pap(dims(N_h=6, H_kv=2, block_size=16, max_blocks=4, num_blocks=8)), U),
    # more than 32 copies or 192 entries take two launches; every argument is
    # still checked before the first of them is enqueued
    ("paged step 33 copies, null v_hat", pap(pdims(), copies=pairs(*([1, 2, 0] * 33)), nc=33, vh=N), E),
    ("paged step 33 copies, rope base", pap(pdims(), copies=pairs(*([1, 2, 0] * 33)), nc=33, base=1.0), E),
    ("paged step 200 entries, capacity", pap(pdims(), entries=pairs(*([0, 3] * 200)), ne=200, max_pos=16 * 4 + 16), CAP),
    ("paged step 200 entries, null q", pap(pdims(), entries=pairs(*([0, 3] * 200)), ne=200, q=N), E),
    # sizes the kernels' 32-bit quantities cannot address
    ("paged table slots past int32", proj(dims(B=65535, block_size=1, max_blocks=40000, num_blocks=8)), U),
    ("paged rows a sequence past int32", proj(dims(block_size=1 << 16, max_blocks=1 << 16, num_blocks=8)), U),
    ("contiguous unit plane of 2^32 bytes", dec(dims(k=128, n_cap=1 << 24)), U),
    ("contiguous unit value plane of 2^32 bytes (k_v wider)", proj(dims(k=8, k_v=16, n_cap=1 << 27)), U),
]
def sread(buf=0x1000, nbytes=1 << 20, waves=64, sink=0x2000):
    return L.swan_measure_stream_read(C.c_void_p(buf) if buf else None, nbytes, waves,
                                      C.c_void_p(sink) if sink else None, st)
cases += [
    ("stream read null buffer", sread(buf=0), E),
    ("stream read null sink", sread(sink=0), E),
    ("stream read misaligned", sread(buf=0x1008), E),
    ("stream read 0 bytes", sread(nbytes=0), E),
    ("stream read odd bytes", sread(nbytes=1000), E),
    ("stream read 0 waves", sread(waves=0), E),
    ("stream read too many waves", sread(waves=(1 << 20) + 1), E),
]
def mrate(waves=64, iters=16, sink=0x2000):
    return L.swan_measure_mfma_f64(C.c_double(1.0), waves, iters, C.c_void_p(sink) if sink else None, st)
cases += [
    ("mfma rate null sink", mrate(sink=0), E),
    ("mfma rate 0 waves", mrate(waves=0), E),
    ("mfma rate too many waves", mrate(waves=(1 << 20) + 1), E),
    ("mfma rate 0 iters", mrate(iters=0), E),
    ("mfma rate iters not a multiple of 4", mrate(iters=6), E),
    ("mfma rate too many iters", mrate(iters=(1 << 20) + 4), E),
]
def noalloc(d, c=cache, max_pos=50, **kw):
    a = dict(pos=F, qh=F, oh=F); a.update(kw)
    return L.swan_decode_attn_noalloc(C.byref(d), C.byref(c), a['pos'], max_pos, a['qh'], a['oh'], st)
cases += [
    ("noalloc null q_hat", noalloc(dims(), qh=N), E),
    ("noalloc null cache plane", noalloc(dims(), c=nocache), E),
    ("noalloc capacity", noalloc(dims(), max_pos=100 + 16), CAP),
    # partials of 300k-row units at 64 work rows a wave: ~39 MB, beyond the 16 MiB scratch
    ("noalloc plan beyond the scratch", noalloc(dims(split_tokens=64, n_cap=300000), max_pos=300000), CAP),
]
bad = [(n, got, want) for n, got, want in cases if got != want]
for n, got, want in bad: print("MISMATCH", n, got, want)
print("OK" if not bad else "FAIL", len(cases))
msg = L.swan_last_error().decode()
assert msg, "no error message recorded"
'''


def test_validation_errors_before_any_launch():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + ERROR_CASES], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().splitlines()[-1].startswith("OK"), r.stdout


def test_status_strings():
    L = S.lib()
    assert L.swan_status_str(0) == b"SWAN_OK"
    assert L.swan_status_str(3) == b"SWAN_ERR_CAPACITY"
    with pytest.raises(S.SwanError) as e:
        S.swan_cache_bytes(S.make_dims(1, 1, 1, 0, 32, d_h=64))
    assert e.value.status == S.SWAN_ERR_UNSUPPORTED and "d_h" in str(e.value)
