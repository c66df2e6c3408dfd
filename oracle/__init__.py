"""fp64 CPU oracle of the causal dot product -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The product library
(``prefix_sum_causal_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, compiled with
gcc).  This module only builds that file, marshals numpy arrays to it and
defines the error metric the parity tests use.

Method (causal dot product of "Transformers are RNNs", Algorithm 1, as named in
the opening post of "Dot Product Computes Wrong Values", triton-lang/triton
issue 217): per (n, h) slice, S_i = S_{i-1} + k_i v_i^T and out_i = q_i^T S_i,
inclusive of token i (the state is updated before the row is read in the loop
excerpt later on that page).  The normalised form divides by
phi(q_i) . sum_{j<=i} phi(k_j) + eps with phi = elu + 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile ``src`` into the shared library ``out`` with gcc (portable -O2,
    no host-specific instruction set, so the library runs on any x86-64 host)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def _as_f32(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(_f32p)


def _ptr64(a: np.ndarray):
    return a.ctypes.data_as(_f64p)


class Oracle:
    """ctypes front end of one compiled copy of ``oracle.c``."""

    def __init__(self, libpath: str = LIB):
        self.lib = ctypes.CDLL(libpath)
        L = self.lib
        dims = [_i64, _i64, _i64, _i64]
        L.oracle_fwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _f64p] + dims
        L.oracle_fwd_brute.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p] + dims
        L.oracle_linattn.argtypes = ([_f32p] * 5 + [_f64p] * 3 + dims + [ctypes.c_double, ctypes.c_int])
        L.oracle_linattn_brute.argtypes = ([_f32p] * 5 + [_f64p] + dims + [ctypes.c_double, ctypes.c_int])
        for name in ("oracle_bwd", "oracle_bwd_brute"):
            getattr(L, name).argtypes = [_f32p] * 5 + [_f64p] * 4 + dims
        for name in ("oracle_fwd", "oracle_fwd_brute", "oracle_linattn", "oracle_linattn_brute", "oracle_bwd",
                     "oracle_bwd_brute"):
            getattr(L, name).restype = None
        L.oracle_linattn_bwd.argtypes = [_f32p] * 6 + [_f64p] * 5 + dims + [ctypes.c_double, ctypes.c_int]
        L.oracle_linattn_bwd.restype = None
        L.oracle_state.argtypes = [_f32p, _f32p, _f64p] + dims
        L.oracle_state.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int

    # -- shape helpers -----------------------------------------------------
    @staticmethod
    def _dims(Q, V):
        if Q.ndim < 2 or V.ndim != Q.ndim or Q.shape[:-1] != V.shape[:-1]:
            raise ValueError("Q is [..., L, E] and V is [..., L, M] with equal leading dims")
        L, E = Q.shape[-2:]
        M = V.shape[-1]
        NH = int(np.prod(Q.shape[:-2], dtype=np.int64)) if Q.ndim > 2 else 1
        return NH, L, E, M

    @staticmethod
    def _opt32(x, shape):
        """An optional float input of the given shape (None -> NULL)."""
        if x is None:
            return None, None
        a = _as_f32(x)
        if a.shape != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
        return a, _ptr32(a)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # -- forward -------------------------------------------------------------
    def _prep(self, Q, K, V):
        Q, K, V = _as_f32(Q), _as_f32(K), _as_f32(V)
        if K.shape != Q.shape:
            raise ValueError("K must have Q's shape")
        return (Q, K, V) + self._dims(Q, V)

    def fwd(self, Q, K, V, S0=None, return_state: bool = False):
        """out_i = q_i^T S_i with S_i = S0 + sum_{j<=i} k_j v_j^T (O(L)
        recurrence; S0 = 0 when None).  With return_state also the final
        state S_{L-1}, shape [..., E, M]."""
        Q, K, V, NH, L, E, M = self._prep(Q, K, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        out = np.empty(V.shape, dtype=np.float64)
        Sf = np.empty(Q.shape[:-2] + (E, M), dtype=np.float64)
        self.lib.oracle_fwd(_ptr32(Q), _ptr32(K), _ptr32(V), p0, _ptr64(out), _ptr64(Sf), NH, L, E, M)
        return (out, Sf) if return_state else out

    def fwd_brute(self, Q, K, V, S0=None) -> np.ndarray:
        """out_i = q_i^T S0 + sum_{j<=i} (q_i.k_j) v_j (O(L^2) masked brute force)."""
        Q, K, V, NH, L, E, M = self._prep(Q, K, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        out = np.empty(V.shape, dtype=np.float64)
        self.lib.oracle_fwd_brute(_ptr32(Q), _ptr32(K), _ptr32(V), p0, _ptr64(out), NH, L, E, M)
        return out

    def linattn(self, Q, K, V, eps: float = 1e-6, feature_map: int = 1, S0=None, z0=None,
                return_state: bool = False):
        """Normalised causal linear attention (recurrence with running z, from
        S0 and z0, zero when None).  With return_state also (S_{L-1}, z_{L-1})."""
        Q, K, V, NH, L, E, M = self._prep(Q, K, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        zz, pz = self._opt32(z0, Q.shape[:-2] + (E,))
        out = np.empty(V.shape, dtype=np.float64)
        Sf = np.empty(Q.shape[:-2] + (E, M), dtype=np.float64)
        zf = np.empty(Q.shape[:-2] + (E,), dtype=np.float64)
        self.lib.oracle_linattn(_ptr32(Q), _ptr32(K), _ptr32(V), p0, pz, _ptr64(out), _ptr64(Sf), _ptr64(zf),
                                NH, L, E, M, float(eps), int(feature_map))
        return (out, Sf, zf) if return_state else out

    def linattn_brute(self, Q, K, V, eps: float = 1e-6, feature_map: int = 1, S0=None, z0=None) -> np.ndarray:
        """Normalised causal linear attention (masked brute force)."""
        Q, K, V, NH, L, E, M = self._prep(Q, K, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        zz, pz = self._opt32(z0, Q.shape[:-2] + (E,))
        out = np.empty(V.shape, dtype=np.float64)
        self.lib.oracle_linattn_brute(_ptr32(Q), _ptr32(K), _ptr32(V), p0, pz, _ptr64(out), NH, L, E, M,
                                      float(eps), int(feature_map))
        return out

    # -- backward ------------------------------------------------------------
    def _bwd_common(self, fn, Q, K, V, dO, S0, with_dS0):
        Q, K, V, dO = _as_f32(Q), _as_f32(K), _as_f32(V), _as_f32(dO)
        if K.shape != Q.shape or dO.shape != V.shape:
            raise ValueError("K must have Q's shape and dO V's shape")
        NH, L, E, M = self._dims(Q, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        dQ = np.empty(Q.shape, dtype=np.float64)
        dK = np.empty(Q.shape, dtype=np.float64)
        dV = np.empty(V.shape, dtype=np.float64)
        dS0 = np.empty(Q.shape[:-2] + (E, M), dtype=np.float64)
        fn(_ptr32(Q), _ptr32(K), _ptr32(V), _ptr32(dO), p0, _ptr64(dQ), _ptr64(dK), _ptr64(dV), _ptr64(dS0),
           NH, L, E, M)
        return (dQ, dK, dV, dS0) if with_dS0 else (dQ, dK, dV)

    def bwd(self, Q, K, V, dO, S0=None, with_dS0: bool = False):
        """(dQ, dK, dV[, dS0]) by a forward sweep of S (from S0) and a reverse
        sweep of R; dS0 = sum_i q_i dO_i^T is the gradient of the initial state."""
        return self._bwd_common(self.lib.oracle_bwd, Q, K, V, dO, S0, with_dS0)

    def bwd_brute(self, Q, K, V, dO, S0=None, with_dS0: bool = False):
        """(dQ, dK, dV[, dS0]) from the O(L^2) double sum."""
        return self._bwd_common(self.lib.oracle_bwd_brute, Q, K, V, dO, S0, with_dS0)

    def linattn_bwd(self, Q, K, V, dO, eps: float = 1e-6, feature_map: int = 1, S0=None, z0=None):
        """Gradients (dQ, dK, dV, dS0, dz0) of sum(out * dO) for the
        normalised form out = linattn(Q, K, V, eps, feature_map, S0, z0), with
        respect to the raw Q and K (through phi), V and the initial states."""
        Q, K, V, dO = _as_f32(Q), _as_f32(K), _as_f32(V), _as_f32(dO)
        if K.shape != Q.shape or dO.shape != V.shape:
            raise ValueError("K must have Q's shape and dO V's shape")
        NH, L, E, M = self._dims(Q, V)
        s0, p0 = self._opt32(S0, Q.shape[:-2] + (E, M))
        zz, pz = self._opt32(z0, Q.shape[:-2] + (E,))
        dQ = np.empty(Q.shape, dtype=np.float64)
        dK = np.empty(Q.shape, dtype=np.float64)
        dV = np.empty(V.shape, dtype=np.float64)
        dS0 = np.empty(Q.shape[:-2] + (E, M), dtype=np.float64)
        dz0 = np.empty(Q.shape[:-2] + (E,), dtype=np.float64)
        self.lib.oracle_linattn_bwd(_ptr32(Q), _ptr32(K), _ptr32(V), _ptr32(dO), p0, pz, _ptr64(dQ), _ptr64(dK),
                                    _ptr64(dV), _ptr64(dS0), _ptr64(dz0), NH, L, E, M, float(eps),
                                    int(feature_map))
        return dQ, dK, dV, dS0, dz0

    def state(self, K, V) -> np.ndarray:
        """Final state sum_j k_j v_j^T per slice, shape [..., E, M]."""
        K, V = _as_f32(K), _as_f32(V)
        NH, L, E, M = self._dims(K, V)
        S = np.empty(K.shape[:-2] + (E, M), dtype=np.float64)
        self.lib.oracle_state(_ptr32(K), _ptr32(V), _ptr64(S), NH, L, E, M)
        return S


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from this directory's ``oracle.c`` (built on first use
    when no library is present)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB):
            build()
        _DEFAULT = Oracle(LIB)
    return _DEFAULT


def build_variant(source_text: str, workdir: str | None = None) -> Oracle:
    """Compile a modified copy of the oracle source (used by the tests that
    plant mistakes in the oracle to show that the pins catch them)."""
    d = workdir or tempfile.mkdtemp(prefix="oracle_variant_")
    src = os.path.join(d, "variant.c")
    with open(src, "w") as f:
        f.write(source_text)
    return Oracle(build(src, os.path.join(d, "libvariant.so")))


def max_rel_err(x, ref) -> float:
    """max |x - ref| / max |ref| over the whole tensor, in fp64 (the parity
    metric; 0 when both are all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.max(np.abs(x - ref))) if x.size else 0.0
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
