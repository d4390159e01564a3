"""Opt-in checks of the device-side contracts (GDN_CHECK_CONTRACTS=1): a bad cu_seqlens or
repeated slots come back as GDN_ERR_SHAPE with nothing launched, and valid inputs give the
same results as with the checks off (GPU: the checks copy the index arrays from the
device). Every bad input here is rejected on the host before any kernel runs."""

import numpy as np
import pytest

import workloads
from tests._util import prefill_to_dev, to_host_f64

pytestmark = pytest.mark.gpu

GDN_ERR_SHAPE = 2


def _prefill(x, cu):
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    fin = torch.empty((x.num_seqs, x.h_v, 128, 128), dtype=torch.float32, device="cuda")
    o = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, x.scale,
                              initial_state=d["s0"], final_state=fin)
    torch.cuda.synchronize()
    return to_host_f64(o), to_host_f64(fin)


def test_prefill_contracts(monkeypatch):
    import torch
    import linear_attention_recurrence_amd as gdn
    x = workloads.make_prefill([70, 0, 33], h_qk=1, h_v=2, with_initial_state=True, seed=180)
    good = torch.tensor(x.cu_seqlens, dtype=torch.int32, device="cuda")
    o_off, f_off = _prefill(x, good)
    monkeypatch.setenv("GDN_CHECK_CONTRACTS", "1")
    o_on, f_on = _prefill(x, good)
    np.testing.assert_array_equal(o_on, o_off)
    np.testing.assert_array_equal(f_on, f_off)
    T = int(x.cu_seqlens[-1])
    for bad in ([1, 71, 71, T], [0, 71, 70, T], [0, 70, 70, T - 1]):   # start, order, end
        with pytest.raises(gdn.GdnError) as e:
            _prefill(x, torch.tensor(bad, dtype=torch.int32, device="cuda"))
        assert e.value.status == GDN_ERR_SHAPE, bad
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_conv_prep(torch.zeros((T, 4 * 128), dtype=torch.bfloat16, device="cuda"),
                          torch.zeros((4 * 128, 4), dtype=torch.float32, device="cuda"),
                          torch.tensor([0, 71, 70, T], dtype=torch.int32, device="cuda"),
                          1, 2, 128, 128, 1.0)
    assert e.value.status == GDN_ERR_SHAPE


def test_decode_slot_contracts(monkeypatch):
    import torch
    import linear_attention_recurrence_amd as gdn
    rng = np.random.Generator(np.random.PCG64(181))
    N = 3
    q = torch.from_numpy(rng.standard_normal((N, 1, 128)).astype(np.float32) * 0.05).cuda()
    k = torch.from_numpy(rng.standard_normal((N, 1, 128)).astype(np.float32) * 0.05).cuda()
    v = torch.from_numpy(rng.standard_normal((N, 2, 128)).astype(np.float32)).cuda()
    g = torch.full((N, 2), -0.1, dtype=torch.float32, device="cuda")
    b = torch.full((N, 2), 0.5, dtype=torch.float32, device="cuda")
    pool0 = torch.from_numpy(rng.standard_normal((5, 2, 128, 128)).astype(np.float32) * 0.02).cuda()
    slots = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
    p_off = pool0.clone()
    o_off = gdn.gdn_decode_step(q, k, v, g, b, p_off, 1.0, state_slots=slots)
    monkeypatch.setenv("GDN_CHECK_CONTRACTS", "1")
    p_on = pool0.clone()
    o_on = gdn.gdn_decode_step(q, k, v, g, b, p_on, 1.0, state_slots=slots)
    torch.cuda.synchronize()
    assert torch.equal(o_on, o_off) and torch.equal(p_on, p_off)
    for bad in ([4, 0, 4], [1, -1, 2]):
        pool = pool0.clone()
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_decode_step(q, k, v, g, b, pool, 1.0,
                                state_slots=torch.tensor(bad, dtype=torch.int32, device="cuda"))
        assert e.value.status == GDN_ERR_SHAPE, bad
        torch.cuda.synchronize()
        assert torch.equal(pool, pool0)   # nothing written
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_channel_decay_decode_step(
                q, k, v, torch.full((N, 2, 128), -0.1, dtype=torch.float32, device="cuda"), b,
                pool, 1.0, state_slots=torch.tensor(bad, dtype=torch.int32, device="cuda"))
        assert e.value.status == GDN_ERR_SHAPE, bad
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_verify_step(q.reshape(N, 1, 1, 128).contiguous(), k.reshape(N, 1, 1, 128).contiguous(),
                            v.reshape(N, 1, 2, 128).contiguous(), g.reshape(N, 1, 2).contiguous(),
                            b.reshape(N, 1, 2).contiguous(), pool0.clone(), 1.0,
                            state_slots=torch.tensor([0, 0, 1], dtype=torch.int32, device="cuda"))
    assert e.value.status == GDN_ERR_SHAPE


def test_log_decay_contract(monkeypatch):
    """A log-decay that is positive, infinite or NaN breaks the contract alpha = exp(g) in
    (0, 1]; with the checks on, prefill and decode reject it with nothing written."""
    import torch
    import linear_attention_recurrence_amd as gdn
    x = workloads.make_prefill([70, 33], h_qk=1, h_v=2, with_initial_state=True, seed=182)
    monkeypatch.setenv("GDN_CHECK_CONTRACTS", "1")
    d = prefill_to_dev(x)
    for bad in (0.25, float("inf"), float("-inf"), float("nan")):
        g = d["g"].clone()
        g[40, 1] = bad
        fin = torch.full((2, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda")
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], g, d["beta"], d["cu"], x.scale,
                                  initial_state=d["s0"], final_state=fin)
        assert e.value.status == GDN_ERR_SHAPE, bad
        torch.cuda.synchronize()
        assert bool((fin == 7.0).all())
        pool = d["s0"].clone()
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_decode_step(d["q"][:2], d["k"][:2], d["v"][:2], g[40:42], d["beta"][:2],
                                pool, x.scale)
        assert e.value.status == GDN_ERR_SHAPE, bad
    g = d["g"].clone()
    g[5, 0] = 0.0                      # alpha = 1 is inside the contract
    gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], g, d["beta"], d["cu"], x.scale,
                          initial_state=d["s0"])
    torch.cuda.synchronize()
