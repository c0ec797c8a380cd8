"""ctypes wrapper of the float64 CPU oracle (``swan_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

Everything here is float64 numpy; values the method stores in its fp16 cache
are carried as binary16-exact doubles.  The cache is kept in *logical* layout
(sparse row t = token t of the sequence), so a paged GPU cache is compared by
reading it through its block table.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "swan_oracle.c")
LIB = os.path.join(HERE, "libswan_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _declare(C.CDLL(LIB))
    return _lib


_pd = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_pu8 = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_pl = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i, _l, _d = C.c_int, C.c_long, C.c_double


def _declare(L):
    L.so_round_f16.argtypes = [_d]
    L.so_round_f16.restype = _d
    L.so_round_f16_array.argtypes = [_l, _pd, _pd]
    L.so_round_e4m3.argtypes = [_d]
    L.so_round_e4m3.restype = _d
    L.so_round_e4m3_array.argtypes = [_l, _pd, _pd]
    L.so_rope.argtypes = [_i, _pd, _d, _d, _pd]
    L.so_project.argtypes = [_i, _pd, _d, _d, _pd, _pd]
    L.so_prune.argtypes = [_i, _i, _pd, _pu8, _pd]
    L.so_attend.argtypes = [_i, _i, _pd, _l, _i, _pu8, _pd, _i, _pu8, _pd, _l, _pd, _pd, _pd, _pd]
    L.so_prefill.argtypes = [_i, _i, _i, _i, _i, _i, _l, _l, _pl, _pd, _pd, _pd, _d,
                             _pu8, _pd, _pu8, _pd, _pd, _pd, _i, _i]
    L.so_prefill.restype = _i
    L.so_project_batch.argtypes = [_i, _i, _i, _i, _pd, _pd, _pl, _pd, _d, _pd, _pd]
    L.so_append_batch.argtypes = [_i, _i, _i, _i, _i, _i, _l, _pl, _pd, _pd, _pu8, _pd, _pu8, _pd, _pd, _pd, _i]
    L.so_append_batch.restype = _i
    L.so_decode_batch.argtypes = [_i, _i, _i, _i, _i, _i, _i, _l, _pl, _pd, _pu8, _pd, _pu8, _pd, _pd, _pd, _pd,
                                  _i]
    L.so_step.argtypes = [_i, _i, _i, _i, _i, _i, _i, _l, _pl, _pd, _pd, _pd, _pd, _d,
                          _pu8, _pd, _pu8, _pd, _pd, _pd, _pd, _pd, _pd, _i, _i]
    L.so_step.restype = _i
    return L


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------

def round_f16(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    lib().so_round_f16_array(x.size, x.reshape(-1), y.reshape(-1))
    return y


def round_e4m3(x) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to even, saturating at +-448)."""
    x = _f64(x)
    y = np.empty_like(x)
    lib().so_round_e4m3_array(x.size, x.reshape(-1), y.reshape(-1))
    return y


def rope(x, pos: float, base: float = 10000.0) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    lib().so_rope(x.shape[-1], x, float(pos), float(base), y)
    return y


def project(x, pos: float, P, base: float = 10000.0) -> np.ndarray:
    x, P = _f64(x), _f64(P)
    y = np.empty_like(x)
    lib().so_project(x.shape[-1], x, float(pos), float(base), P, y)
    return y


def prune(x, k: int):
    """(idx uint8 [k], val float64 [k]) of the magnitude top-k of x."""
    x = _f64(x)
    idx = np.zeros(k, np.uint8)
    val = np.zeros(k, np.float64)
    lib().so_prune(x.shape[-1], k, x, idx, val)
    return idx, val


def attend(qhat, kidx, kval, vidx, vval, kd, vd) -> np.ndarray:
    """Hybrid attention of one unit: qhat [g][d]; sparse key rows kidx/kval
    [n][k] and value rows vidx/vval [n][kv] (n may be 0); dense rows kd/vd
    [nd][d] (nd may be 0).  Returns out [g][d] (float64)."""
    qhat = _f64(np.atleast_2d(qhat))
    g, d = qhat.shape
    kval, vval = _f64(kval), _f64(vval)
    n, k = kval.shape
    kv = vval.shape[1]
    kd, vd = _f64(kd).reshape(-1, d), _f64(vd).reshape(-1, d)
    nd = kd.shape[0]
    # the C side never reads past n / nd rows; pad empty arrays to one row
    pad = lambda a, cols, dt: a if a.shape[0] else np.zeros((1, cols), dt)
    kidx = pad(np.ascontiguousarray(kidx, np.uint8).reshape(n, k), k, np.uint8)
    vidx = pad(np.ascontiguousarray(vidx, np.uint8).reshape(n, kv), kv, np.uint8)
    kval, vval = pad(kval, k, np.float64), pad(vval, kv, np.float64)
    kd, vd = pad(kd, d, np.float64), pad(vd, d, np.float64)
    out = np.zeros((g, d))
    scratch = np.zeros(n + nd + 1)
    lib().so_attend(d, g, qhat, n, k, kidx, kval, kv, vidx, vval, nd, kd, vd, out, scratch)
    return out


# ---------------------------------------------------------------------------
# batched logical cache
# ---------------------------------------------------------------------------

class OracleCache:
    """The hybrid cache of a batch in logical layout (float64, binary16-exact
    values; with value_format 1 the sparse values are E4M3-exact): key rows
    [B][H][ncap][k], value rows [B][H][ncap][k_v] (k_v = k unless given) and
    dense buffer [B][H][R][d]."""

    def __init__(self, B: int, N_h: int, H_kv: int, d: int, R: int, k: int, ncap: int, value_format: int = 0,
                 k_v: int | None = None):
        self.B, self.N_h, self.H_kv, self.d, self.R, self.k, self.ncap = B, N_h, H_kv, d, R, k, ncap
        self.k_v = int(k_v) if k_v else k
        self.value_format = int(value_format)
        self.kidx = np.zeros((B, H_kv, ncap, k), np.uint8)
        self.vidx = np.zeros((B, H_kv, ncap, self.k_v), np.uint8)
        self.kval = np.zeros((B, H_kv, ncap, k))
        self.vval = np.zeros((B, H_kv, ncap, self.k_v))
        self.ringk = np.zeros((B, H_kv, max(R, 1), d))
        self.ringv = np.zeros_like(self.ringk)

    @classmethod
    def for_workload(cls, w, ncap: int | None = None):
        return cls(w.B, w.N_h, w.H_kv, w.d_h, w.R, w.k, w.n_cap() if ncap is None else ncap,
                   getattr(w, "value_format", 0), getattr(w, "k_v", 0) or None)

    def _state(self):
        return (self.kidx, self.kval, self.vidx, self.vval, self.ringk, self.ringv)

    def prefill(self, Kraw, Vraw, T, P, base: float = 10000.0, nthreads: int | None = None):
        """Kraw, Vraw [B][H][Tmax][d]; T[b] prefilled tokens (positions 0..T-1)."""
        Kraw, Vraw = _f64(Kraw), _f64(Vraw)
        T = np.ascontiguousarray(T, np.int64)
        err = lib().so_prefill(self.B, self.H_kv, self.d, self.R, self.k, self.k_v, self.ncap, Kraw.shape[2], T,
                               Kraw, Vraw, _f64(P), float(base), *self._state(),
                               nthreads or default_threads(), self.value_format)
        if err:
            raise ValueError("sparse capacity exceeded in prefill")

    def project(self, q, kraw, pos, P, base: float = 10000.0):
        qhat = np.zeros((self.B, self.N_h, self.d))
        khat = np.zeros((self.B, self.H_kv, self.d))
        lib().so_project_batch(self.B, self.N_h, self.H_kv, self.d, _f64(q), _f64(kraw),
                               np.ascontiguousarray(pos, np.int64), _f64(P), float(base), qhat, khat)
        return qhat, khat

    def append(self, khat, vhat, pos):
        err = lib().so_append_batch(self.B, self.H_kv, self.d, self.R, self.k, self.k_v, self.ncap,
                                    np.ascontiguousarray(pos, np.int64), _f64(khat), _f64(vhat), *self._state(),
                                    self.value_format)
        if err:
            raise ValueError("sparse capacity exceeded in append")

    def decode(self, qhat, pos, nthreads: int | None = None):
        out = np.zeros((self.B, self.N_h, self.d))
        lib().so_decode_batch(self.B, self.N_h, self.H_kv, self.d, self.R, self.k, self.k_v, self.ncap,
                              np.ascontiguousarray(pos, np.int64), _f64(qhat), *self._state(), out,
                              nthreads or default_threads())
        return out

    def step(self, q, kraw, vnew, pos, P, base: float = 10000.0, nthreads: int | None = None):
        """Whole step; returns (qhat, khat_rounded, out)."""
        qhat = np.zeros((self.B, self.N_h, self.d))
        khat = np.zeros((self.B, self.H_kv, self.d))
        out = np.zeros((self.B, self.N_h, self.d))
        err = lib().so_step(self.B, self.N_h, self.H_kv, self.d, self.R, self.k, self.k_v, self.ncap,
                            np.ascontiguousarray(pos, np.int64), _f64(q), _f64(kraw), _f64(vnew), _f64(P),
                            float(base), *self._state(), qhat, khat, out, nthreads or default_threads(),
                            self.value_format)
        if err:
            raise ValueError("sparse capacity exceeded in step")
        return qhat, khat, out

    def copy(self) -> "OracleCache":
        c = OracleCache.__new__(OracleCache)
        c.__dict__.update({k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in self.__dict__.items()})
        return c

    # views in the storage formats the GPU cache uses (for comparisons)
    def sparse_f16(self, b: int, h: int, n: int):
        """(kidx, kval fp16, vidx, vval fp16) rows 0..n-1 of unit (b, h)."""
        return (self.kidx[b, h, :n], self.kval[b, h, :n].astype(np.float16),
                self.vidx[b, h, :n], self.vval[b, h, :n].astype(np.float16))

    def ring_f16(self):
        return self.ringk.astype(np.float16), self.ringv.astype(np.float16)
