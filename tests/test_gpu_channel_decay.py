"""The per-channel form (one decay per value channel, correction from the state before the
decay): gdn_channel_decay_prefill and gdn_channel_decay_decode_step against the fp64 oracle,
and decode steps against prefill (GPU)."""

import numpy as np
import pytest

import oracle
import workloads
from tests._util import check_outputs, check_state, prefill_to_dev, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _oracle(x, g, heads=None):
    ref_o, ref_s, _ = oracle.recurrence_channel(x.as_f64("q"), x.as_f64("k"), x.as_f64("v"),
                                                g.astype(np.float64), x.as_f64("beta"),
                                                x.cu_seqlens, x.scale,
                                                initial_state=x.as_f64("initial_state")
                                                if x.initial_state is not None else None)
    return ref_o, ref_s


def _run_prefill(x, g):
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    N = x.num_seqs
    fin = torch.full((N, x.h_v, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    o = gdn.gdn_channel_decay_prefill(d["q"], d["k"], d["v"], to_dev(g), d["beta"], d["cu"], x.scale,
                                      initial_state=d["s0"], final_state=fin)
    torch.cuda.synchronize()
    return to_host_f64(o), to_host_f64(fin)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_channel_prefill_varlen(io):
    """Lengths 0, 1, 17, 64 and 150 (a zero-length sequence keeps its initial state)."""
    x = workloads.make_prefill([0, 1, 17, 64, 150], h_qk=2, h_v=4, io_dtype=io,
                               with_initial_state=True, seed=150)
    g = workloads.channel_log_alpha(x.total_tokens, 4, 128, seed=151)
    o, fin = _run_prefill(x, g)
    ref_o, ref_s = _oracle(x, g)
    res_o = check_outputs(o, ref_o, "channel prefill %s" % io)
    res_s = check_state(fin, ref_s, "channel prefill %s" % io)
    if io == "f32":
        assert res_o[1] < 1e-5 and res_s < 1e-5
    np.testing.assert_array_equal(fin[0], x.initial_state[0].astype(np.float64))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_channel_prefill_many_pairs(io):
    """More than 64 (sequence, V head) pairs: the prefill takes its other shape (8 rows per
    wave, 4 tokens in flight). Lengths below, at and past multiples of the ring depth."""
    x = workloads.make_prefill([0, 3, 40, 130, 7], h_qk=16, h_v=32, io_dtype=io,
                               with_initial_state=True, seed=156)
    g = workloads.channel_log_alpha(x.total_tokens, 32, 128, seed=157)
    o, fin = _run_prefill(x, g)
    ref_o, ref_s = _oracle(x, g)
    res_o = check_outputs(o, ref_o, "channel prefill 160 pairs %s" % io)
    res_s = check_state(fin, ref_s, "channel prefill 160 pairs %s" % io)
    if io == "f32":
        assert res_o[1] < 1e-5 and res_s < 1e-5
    np.testing.assert_array_equal(fin[0], x.initial_state[0].astype(np.float64))


def test_channel_prefill_shape_boundary():
    """64 (sequence, V head) pairs take the 4-row shape and 65 the 8-row one: the same two
    sequences run alone (2 x 32 pairs) and beside a third (3 x 32 pairs) agree to rounding,
    and both match the oracle."""
    lens = [150, 77]
    x3 = workloads.make_prefill(lens + [33], h_qk=16, h_v=32, with_initial_state=True, seed=158)
    g3 = workloads.channel_log_alpha(x3.total_tokens, 32, 128, seed=159)
    T2 = sum(lens)
    x2 = workloads.PrefillInputs(q=x3.q[:T2], k=x3.k[:T2], v=x3.v[:T2], g=x3.g[:T2],
                                 beta=x3.beta[:T2], cu_seqlens=x3.cu_seqlens[:3].copy(),
                                 initial_state=x3.initial_state[:2], scale=x3.scale,
                                 io_dtype="bf16")
    o3, f3 = _run_prefill(x3, g3)
    o2, f2 = _run_prefill(x2, g3[:T2])
    check_outputs(o2, o3[:T2], "2 vs 3 sequences")
    check_state(f2, f3[:2], "2 vs 3 sequences")
    ref_o, ref_s = _oracle(x2, g3[:T2])
    check_outputs(o2, ref_o, "64 pairs")
    check_state(f2, ref_s, "64 pairs")
    assert np.isfinite(o3).all()


def test_channel_prefill_model_size():
    """B = 1, T = 1024, 16 QK / 32 V heads, bf16, S0 ~ N(0, 0.02): every head against the oracle."""
    x = workloads.make_prefill([1024], with_initial_state=True, seed=152)
    g = workloads.channel_log_alpha(1024, seed=153)
    o, fin = _run_prefill(x, g)
    ref_o, ref_s = _oracle(x, g)
    check_outputs(o, ref_o, "channel prefill T=1024")
    check_state(fin, ref_s, "channel prefill T=1024")


def test_channel_decode_equals_prefill():
    """Token-by-token decode over a permuted pool agrees with the prefill of the same tokens
    (the two kernels sum the per-row products in different orders, so to rounding), and both
    match the oracle."""
    import torch
    import linear_attention_recurrence_amd as gdn
    T, N = 12, 3
    x = workloads.make_prefill([T] * N, h_qk=1, h_v=2, with_initial_state=True, seed=154)
    g = workloads.channel_log_alpha(T * N, 2, 128, seed=155)
    o_p, fin_p = _run_prefill(x, g)
    d = prefill_to_dev(x)
    slots = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
    pool = torch.zeros((5, 2, 128, 128), dtype=torch.float32, device="cuda")
    pool[slots.long()] = d["s0"]
    gd = to_dev(g)
    rows = lambda t: torch.arange(N, device="cuda") * T + t
    outs = []
    for t in range(T):
        r = rows(t)
        outs.append(gdn.gdn_channel_decay_decode_step(
            d["q"][r].contiguous(), d["k"][r].contiguous(), d["v"][r].contiguous(), gd[r].contiguous(),
            d["beta"][r].contiguous(), pool, x.scale, state_slots=slots))
    torch.cuda.synchronize()
    o_d = np.stack([to_host_f64(o_) for o_ in outs], axis=1).reshape(N * T, 2, 128)
    fin_d = to_host_f64(pool[slots.long()])
    check_outputs(o_d, o_p, "channel decode vs prefill")
    check_state(fin_d, fin_p, "channel decode vs prefill")
    ref_o, ref_s = _oracle(x, g)
    check_outputs(o_d, ref_o, "channel decode")
    check_state(fin_d, ref_s, "channel decode")
    check_outputs(o_p, ref_o, "channel prefill")
    check_state(fin_p, ref_s, "channel prefill")
