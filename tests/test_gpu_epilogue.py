"""The output epilogue (per-head RMS norm with the zero-centred scale, then the output gate):
gdn_gated_rmsnorm against the fp64 oracle (GPU)."""

import numpy as np
import pytest

import oracle
import workloads
from tests._util import to_dev, to_host_f64

pytestmark = pytest.mark.gpu

def _inputs(rows, h_v, io, seed):
    return workloads.epilogue_inputs(rows, h_v, io_dtype=io, seed=seed)


def _widen(a):
    return workloads.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _check(out, ref, io):
    """bf16: every element within half a bf16 spacing of the fp64 result, plus the fp32
    arithmetic's few-ulp error before that rounding; fp32: 1e-5 relative per element plus
    1e-6 of the vector's largest entry."""
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    err = np.abs(out - ref)
    if io == "bf16":
        spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        bound = 0.5 * spacing + 2e-6 * np.abs(ref) + 1e-7 * scale
    else:
        bound = 1e-5 * np.abs(ref) + 1e-6 * scale
    bad = err > bound
    assert not bad.any(), "%d of %d elements off, worst excess %.3e" % (
        bad.sum(), bad.size, float(np.max((err - bound) / (scale + 1e-30))))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["sigmoid", "silu"])
def test_gated_rmsnorm_against_oracle(io, gate):
    """Ragged vector count (rows x h_v not a multiple of a workgroup's 16 vectors)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    o, z, w = _inputs(37, 5, io, seed=170 + (io == "f32") + 2 * (gate == "silu"))
    eps = 1e-6
    out = gdn.gdn_gated_rmsnorm(to_dev(o), to_dev(z), to_dev(w), eps=eps, gate=gate)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(_widen(o), _widen(z), w.astype(np.float64), eps=eps,
                               gate=oracle.GATE_SILU if gate == "silu" else oracle.GATE_SIGMOID)
    _check(to_host_f64(out), ref, io)


def test_gated_rmsnorm_model_size_in_place():
    """B = 1, T = 4096, 32 V heads, bf16, written over o; a second call over z equals it."""
    import torch
    import linear_attention_recurrence_amd as gdn
    o, z, w = _inputs(4096, 32, "bf16", seed=175)
    ref = oracle.gated_rmsnorm(_widen(o), _widen(z), w.astype(np.float64), eps=1e-6)
    od, zd, wd = to_dev(o), to_dev(z), to_dev(w)
    fresh = gdn.gdn_gated_rmsnorm(od, zd, wd)
    gdn.gdn_gated_rmsnorm(od, zd, wd, out=od)
    torch.cuda.synchronize()
    assert torch.equal(od, fresh)
    _check(to_host_f64(od), ref, "bf16")
    zd2 = to_dev(z)
    gdn.gdn_gated_rmsnorm(to_dev(o), zd2, wd, out=zd2)
    torch.cuda.synchronize()
    assert torch.equal(zd2, fresh)


def test_gated_rmsnorm_edge_cases():
    """Zero read-out (eps keeps it finite: zeros out), a tiny vector, eps = 0 on a nonzero
    vector, gate inputs of +-200 (the gate saturates to 0 and to z), and zero rows."""
    import torch
    import linear_attention_recurrence_amd as gdn
    o = np.zeros((3, 2, 128), dtype=np.float32)
    o[1, 0] = np.linspace(-2, 2, 128)
    o[2, 1] = 1e-20
    z = np.zeros_like(o)
    z[1, 0, :64] = 200.0
    z[1, 0, 64:] = -200.0
    w = np.zeros(128, dtype=np.float32)
    for eps in (1e-6, 0.0):
        out = gdn.gdn_gated_rmsnorm(to_dev(o), to_dev(z), to_dev(w), eps=eps, gate="silu")
        torch.cuda.synchronize()
        got = to_host_f64(out)
        ref = oracle.gated_rmsnorm(o.astype(np.float64), z.astype(np.float64),
                                   w.astype(np.float64), eps=eps, gate=oracle.GATE_SILU)
        if eps > 0:
            # every vector, the all-zero ones included (zeros out)
            assert np.all(np.isfinite(got))
            assert np.all(got[0] == 0.0)
            assert np.allclose(got, ref, rtol=1e-5, atol=1e-12)
        else:
            # without eps only a nonzero vector is defined (an all-zero one is 0/0)
            assert np.all(np.isfinite(got[1, 0]))
            assert np.allclose(got[1, 0], ref[1, 0], rtol=1e-5, atol=1e-6)
    empty = torch.empty((0, 2, 128), dtype=torch.float32, device="cuda")
    gdn.gdn_gated_rmsnorm(empty, empty, to_dev(w))
