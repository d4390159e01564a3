"""Front end parity: gdn_conv_prep against the fp64 oracle, and the packed variable-length
front end + prefill chain (GPU)."""

import numpy as np
import pytest

import oracle
import workloads
from tests._util import (bf16_bits, check_outputs, check_state, oracle_prefill, to_dev,
                         to_host_f64)

pytestmark = pytest.mark.gpu


def _conv_gpu(fe):
    import torch
    import linear_attention_recurrence_amd as gdn
    q, k, v = gdn.gdn_conv_prep(to_dev(fe.mixed), to_dev(fe.conv_weight), to_dev(fe.cu_seqlens),
                                fe.h_qk, fe.h_v, fe.d_k, fe.d_v, fe.q_scale)
    torch.cuda.synchronize()
    return q, k, v


def _check_one_rounding(gpu, ref, label):
    """Each element within one bf16 rounding of the fp64 value (plus fp32 arithmetic)."""
    err = np.abs(gpu - ref)
    bound = 2.0 ** -8 * np.abs(ref) * (1 + 1e-3) + 1e-6
    bad = err > bound
    assert not bad.any(), "%s: %d elements off, worst %.3e" % (label, bad.sum(), (err - bound).max())


def _oracle_conv(fe, seqs=None):
    mixed = workloads.bf16_bits_to_f32(fe.mixed)
    cu = fe.cu_seqlens
    seqs = range(fe.num_seqs) if seqs is None else seqs
    out = {}
    for n in seqs:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        q, k, v = oracle.conv_prep(mixed[t0:t1].astype(np.float64), fe.conv_weight.astype(np.float64),
                                   [0, t1 - t0], fe.h_qk, fe.h_v, fe.d_k, fe.d_v, fe.q_scale)
        out[n] = (q, k, v)
    return out


@pytest.mark.parametrize("lens", [[1], [3, 0, 5], [31, 33, 64], [200, 1, 2, 3, 100]])
def test_conv_prep_small(lens):
    fe = workloads.make_frontend(lens, h_qk=2, h_v=4, seed=60 + len(lens))
    q, k, v = _conv_gpu(fe)
    ref = _oracle_conv(fe)
    for n, (qr, kr, vr) in ref.items():
        t0, t1 = int(fe.cu_seqlens[n]), int(fe.cu_seqlens[n + 1])
        _check_one_rounding(to_host_f64(q[t0:t1]), qr, "q seq %d" % n)
        _check_one_rounding(to_host_f64(k[t0:t1]), kr, "k seq %d" % n)
        _check_one_rounding(to_host_f64(v[t0:t1]), vr, "v seq %d" % n)


@pytest.mark.parametrize("K", [1, 2, 3])
def test_conv_prep_short_kernels(K):
    fe = workloads.make_frontend([40, 9], h_qk=1, h_v=2, conv_kernel=K, seed=70 + K)
    q, k, v = _conv_gpu(fe)
    ref = _oracle_conv(fe)
    for n, (qr, kr, vr) in ref.items():
        t0, t1 = int(fe.cu_seqlens[n]), int(fe.cu_seqlens[n + 1])
        _check_one_rounding(to_host_f64(v[t0:t1]), vr, "v K=%d" % K)
        _check_one_rounding(to_host_f64(k[t0:t1]), kr, "k K=%d" % K)


def test_config4_front_end_and_prefill():
    """64 sequences, lengths uniform in [128, 8192], mixed bf16 [sum T][8192], conv k = 4,
    S0 ~ N(0, 0.02), final states. Stage 1: the front end on three whole sequences against
    the fp64 front end. Stage 2: the recurrence on the GPU's own bf16 q, k, v for those
    sequences (all heads) against the oracle fed the same bits."""
    import torch
    import linear_attention_recurrence_amd as gdn
    fe = workloads.config4()
    cu = fe.cu_seqlens
    lens = np.diff(cu)
    q, k, v = _conv_gpu(fe)
    s0 = to_dev(fe.initial_state)
    fin = torch.empty_like(s0)
    o = gdn.gdn_chunk_prefill(q, k, v, to_dev(fe.g), to_dev(fe.beta), to_dev(cu), 1.0,
                              initial_state=s0, final_state=fin)
    torch.cuda.synchronize()
    seqs = [int(np.argmin(lens)), 0, int(np.argmax(lens))]
    ref = _oracle_conv(fe, seqs)
    for n in seqs:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        qr, kr, vr = ref[n]
        _check_one_rounding(to_host_f64(q[t0:t1]), qr, "q seq %d" % n)
        _check_one_rounding(to_host_f64(k[t0:t1]), kr, "k seq %d" % n)
        _check_one_rounding(to_host_f64(v[t0:t1]), vr, "v seq %d" % n)
    # stage 2: the recurrence on the GPU's own front-end output (scale 1: q is pre-scaled)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    x = workloads.PrefillInputs(q=qb, k=kb, v=vb, g=fe.g, beta=fe.beta, cu_seqlens=cu,
                                initial_state=fe.initial_state, scale=1.0, io_dtype="bf16")
    o_h = to_host_f64(o)
    fin_h = to_host_f64(fin)
    refp = oracle_prefill(x, seqs=seqs)
    for n in seqs:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        o_sel = np.stack([o_h[t0:t1, h] for h in range(32)])
        r_sel = np.stack([refp[(n, h)][0] for h in range(32)])
        check_outputs(o_sel, r_sel, "config4 seq %d" % n)
        check_state(fin_h[n], np.stack([refp[(n, h)][1] for h in range(32)]), "config4 seq %d" % n)
