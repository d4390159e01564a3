"""fp64 CPU oracle for the Gated DeltaNet token mixer (TEST INFRASTRUCTURE ONLY).

This package is the reference the GPU library is checked against. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the library itself never
does, and the two share no code.

* ``gdn_oracle.c``  -- the token loop and the front end in plain fp64 C (see its header for
  the passages each function follows), built here with gcc into ``libgdn_oracle.so``.
* ``brute.py``      -- exact rational arithmetic (Python ``fractions``) of the unrolled
  product form, for tiny cases.

All arrays passed in are float64 numpy arrays holding the exact values the GPU received
(bf16 inputs widened exactly).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math). Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: Optional[str] = None):
    """ctypes handle of a built oracle library (default: the one built from gdn_oracle.c)."""
    lib = ctypes.CDLL(path or _LIB)
    lib.gdn_ref_recurrence.restype = ctypes.c_int
    lib.gdn_ref_recurrence.argtypes = [_D, _D, _D, _D, _D, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, _D, _D, _D, _D,
                                       ctypes.c_int]
    lib.gdn_ref_recurrence_channel.restype = ctypes.c_int
    lib.gdn_ref_recurrence_channel.argtypes = lib.gdn_ref_recurrence.argtypes
    lib.gdn_ref_conv_prep.restype = ctypes.c_int
    lib.gdn_ref_conv_prep.argtypes = [_D, _D, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                      _D, _D, _D, ctypes.c_int]
    lib.gdn_ref_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_ref_gated_rmsnorm.argtypes = [_D, _D, _D, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, ctypes.c_int, _D]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_D)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def recurrence(q, k, v, g, beta, cu_seqlens, scale, initial_state=None,
               want_final=True, want_traj=False, n_threads=None, lib=None):
    """Gated delta rule over a packed batch, fp64.

    q, k: [T][h_qk][d_k]; v: [T][h_v][d_v]; g, beta: [T][h_v]; cu_seqlens: [N+1].
    initial_state: [N][h_v][d_v][d_k] or None (zeros).
    Returns (o [T][h_v][d_v], final_state [N][h_v][d_v][d_k] or None,
             traj [h_v][T][d_v][d_k] or None).
    """
    f = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    q, k, v, g, beta = f(q), f(k), f(v), f(g), f(beta)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, h_qk, d_k = q.shape
    _, h_v, d_v = v.shape
    N = len(cu) - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, h_v) == beta.shape
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0 = None if initial_state is None else f(initial_state)
    if s0 is not None:
        assert s0.shape == (N, h_v, d_v, d_k)
    o = np.zeros((T, h_v, d_v), dtype=np.float64)
    fin = np.zeros((N, h_v, d_v, d_k), dtype=np.float64) if want_final else None
    traj = np.zeros((h_v, T, d_v, d_k), dtype=np.float64) if want_traj else None
    rc = (lib or _load()).gdn_ref_recurrence(_dp(q), _dp(k), _dp(v), _dp(g), _dp(beta),
                                    cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
                                    h_qk, h_v, d_k, d_v, float(scale), _dp(s0), _dp(fin),
                                    _dp(o), _dp(traj),
                                    int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, fin, traj


def recurrence_channel(q, k, v, g, beta, cu_seqlens, scale, initial_state=None,
                       want_final=True, want_traj=False, n_threads=None, lib=None):
    """The per-channel form, fp64: one log-decay per value channel, g [T][h_v][d_v], and the
    correction taken from the state before the decay (code panel of section
    "01 . GatedDeltaNet(config)" of "Qwen3-Next 80B-A3B -- The Evolving Transformer").
    Other arguments and the returned tuple as for recurrence()."""
    f = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    q, k, v, g, beta = f(q), f(k), f(v), f(g), f(beta)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, h_qk, d_k = q.shape
    _, h_v, d_v = v.shape
    N = len(cu) - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, h_v, d_v)
    assert beta.shape == (T, h_v)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0 = None if initial_state is None else f(initial_state)
    if s0 is not None:
        assert s0.shape == (N, h_v, d_v, d_k)
    o = np.zeros((T, h_v, d_v), dtype=np.float64)
    fin = np.zeros((N, h_v, d_v, d_k), dtype=np.float64) if want_final else None
    traj = np.zeros((h_v, T, d_v, d_k), dtype=np.float64) if want_traj else None
    rc = (lib or _load()).gdn_ref_recurrence_channel(
        _dp(q), _dp(k), _dp(v), _dp(g), _dp(beta), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        N, h_qk, h_v, d_k, d_v, float(scale), _dp(s0), _dp(fin), _dp(o), _dp(traj),
        int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, fin, traj


def conv_prep(mixed, conv_weight, cu_seqlens, h_qk, h_v, d_k, d_v, q_scale, eps=1e-12,
              n_threads=None, lib=None):
    """Front end in fp64: causal depthwise conv, SiLU, q/k L2 norm, q scale.

    mixed: [T][2*h_qk*d_k + h_v*d_v] (channels q | k | v, head-major);
    conv_weight: [channels][K] with tap K-1 on the current token.
    Returns q, k [T][h_qk][d_k] and v [T][h_v][d_v].
    """
    x = np.ascontiguousarray(mixed, dtype=np.float64)
    w = np.ascontiguousarray(conv_weight, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, C = x.shape
    assert C == 2 * h_qk * d_k + h_v * d_v and w.shape[0] == C
    q = np.zeros((T, h_qk, d_k)); k = np.zeros((T, h_qk, d_k)); v = np.zeros((T, h_v, d_v))
    rc = (lib or _load()).gdn_ref_conv_prep(_dp(x), _dp(w), int(w.shape[1]),
                                   cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(cu) - 1,
                                   h_qk, h_v, d_k, d_v, float(q_scale), float(eps),
                                   _dp(q), _dp(k), _dp(v), int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return q, k, v


GATE_SIGMOID = 0
GATE_SILU = 1


def gated_rmsnorm(o, z, weight, eps=1e-6, gate=GATE_SIGMOID, lib=None):
    """Output epilogue (gdn_oracle.c, gdn_ref_gated_rmsnorm): per V head, RMS norm over the
    d_v read-out channels with the zero-centred scale (1 + weight) (architecture
    knowledge-base page "Qwen3-Next 80B-A3B", table "Architecture", row "Norm type"), then
    the output gate of the GatedDeltaNet section of the Evolving Transformer page,
    sigmoid(z) or SiLU(z), elementwise.

    o, z: [rows][h_v][d_v] float64; weight: [d_v] float64. Returns out, same shape as o."""
    o = np.ascontiguousarray(o, dtype=np.float64)
    z = np.ascontiguousarray(z, dtype=np.float64)
    weight = np.ascontiguousarray(weight, dtype=np.float64)
    rows, h_v, d_v = o.shape
    assert z.shape == o.shape and weight.shape == (d_v,)
    out = np.empty_like(o)
    L = lib or _load()
    st = L.gdn_ref_gated_rmsnorm(_dp(o), _dp(z), _dp(weight), rows, h_v, d_v, float(eps),
                                 int(gate), _dp(out))
    if st != 0:
        raise ValueError("gated_rmsnorm: unknown gate %r" % (gate,))
    return out
