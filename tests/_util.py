"""Helpers shared by the tests: device transfer of seeded inputs and the parity checks.

Tolerances (floating point, whole tensors): max |o_gpu - o_ref| <= 2e-2,
||o_gpu - o_ref||_F / ||o_ref||_F <= 5e-3, ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-3,
with o_ref and S_ref from the fp64 oracle fed exactly the bits the GPU received.
"""

from __future__ import annotations

import numpy as np

O_MAX_ABS = 2e-2
O_REL_F = 5e-3
S_REL_F = 1e-3


def to_dev(a, dtype=None):
    """numpy -> torch on cuda:0; uint16 arrays are bf16 bit patterns."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def to_host_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_bits(t) -> np.ndarray:
    """bf16 torch tensor -> uint16 numpy bit patterns (exact)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_f(a, b) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / nb if nb > 0 else float(np.linalg.norm(a - b))


def check_outputs(o_gpu, o_ref, label=""):
    d = np.abs(o_gpu - o_ref)
    max_abs = float(d.max()) if d.size else 0.0
    rf = rel_f(o_gpu, o_ref) if d.size else 0.0
    assert max_abs <= O_MAX_ABS, "%s max|do| = %.3e" % (label, max_abs)
    assert rf <= O_REL_F, "%s relF(o) = %.3e" % (label, rf)
    return max_abs, rf


def check_state(s_gpu, s_ref, label=""):
    rf = rel_f(s_gpu, s_ref)
    assert rf <= S_REL_F, "%s relF(S) = %.3e" % (label, rf)
    return rf


def prefill_to_dev(x):
    """workloads.PrefillInputs -> dict of device tensors."""
    import torch
    return dict(q=to_dev(x.q), k=to_dev(x.k), v=to_dev(x.v), g=to_dev(x.g), beta=to_dev(x.beta),
                cu=to_dev(x.cu_seqlens), s0=to_dev(x.initial_state))


def oracle_prefill(x, heads=None, seqs=None, n_threads=None):
    """fp64 oracle on (a subset of) a PrefillInputs batch.

    heads: list of QK heads j; their V heads j*group .. j*group+group-1 are computed.
    seqs: list of sequence indices. Returns dict (n, h) -> (o [T_n][d_v], S [d_v][d_k]).
    """
    import oracle
    h_qk, h_v = x.h_qk, x.h_v
    group = h_v // h_qk
    heads = range(h_qk) if heads is None else heads
    seqs = range(x.num_seqs) if seqs is None else seqs
    q, k, v = x.as_f64("q"), x.as_f64("k"), x.as_f64("v")
    g, b = x.as_f64("g"), x.as_f64("beta")
    s0 = x.as_f64("initial_state")
    heads = list(heads)
    vheads = [j * group + gi for j in heads for gi in range(group)]
    out = {}
    for n in seqs:
        t0, t1 = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        init = None if s0 is None else s0[n:n + 1][:, vheads]
        # the selected heads keep the mapping: V head index i reads QK head index i // group
        o, fin, _ = oracle.recurrence(q[t0:t1][:, heads], k[t0:t1][:, heads], v[t0:t1][:, vheads],
                                      g[t0:t1][:, vheads], b[t0:t1][:, vheads], [0, t1 - t0],
                                      x.scale, initial_state=init, n_threads=n_threads)
        for i, h in enumerate(vheads):
            out[(n, h)] = (o[:, i], fin[0, i])
    return out
