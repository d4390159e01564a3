"""Multi-token verify: gdn_verify_step against successive gdn_decode_step calls (bit for bit)
and against the fp64 oracle (GPU)."""

import numpy as np
import pytest

import oracle
import workloads
from tests._util import check_outputs, check_state, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _seq_major(a):
    """[ring][N][...] -> [N][ring][...] (token t of sequence n is ring entry t)."""
    return np.ascontiguousarray(np.swapaxes(a, 0, 1))


def _inputs(d, io):
    import torch
    dev = dict(q=to_dev(d.q), k=to_dev(d.k), v=to_dev(d.v), g=to_dev(d.g), beta=to_dev(d.beta))
    seq = dict(q=to_dev(_seq_major(d.q)), k=to_dev(_seq_major(d.k)), v=to_dev(_seq_major(d.v)),
               g=to_dev(_seq_major(d.g)), beta=to_dev(_seq_major(d.beta)))
    if io == "f32":
        for x in (dev, seq):
            for name in ("q", "k", "v"):
                x[name] = x[name].to(torch.float32)
    return dev, seq


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("permuted", [False, True])
def test_verify_equals_decode_steps(io, permuted):
    """4 draft tokens for 5 sequences: outputs, the final pool and every snapshot equal, bit for
    bit, those of 4 successive decode steps (untouched pool entries stay as they were)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    n_tok = 4
    d = workloads.make_decode(num_seqs=5, h_qk=2, h_v=4, ring=n_tok, pool_size=9 if permuted else None,
                              permuted_slots=permuted, seed=140)
    dev, seq = _inputs(d, io)
    slots = to_dev(d.slots)
    pool_a = to_dev(d.pool)
    pool_b = to_dev(d.pool)
    snaps = torch.full((5, n_tok, 4, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    o_v = gdn.gdn_verify_step(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"], pool_a, d.scale,
                              state_slots=slots, snapshots=snaps)
    o_d, pools = [], []
    sl = torch.arange(5, device="cuda") if slots is None else slots.long()
    for t in range(n_tok):
        o_d.append(gdn.gdn_decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t],
                                       pool_b, d.scale, state_slots=slots).clone())
        pools.append(pool_b[sl].clone())
    torch.cuda.synchronize()
    for t in range(n_tok):
        assert torch.equal(o_v[:, t], o_d[t]), "output of token %d" % t
        assert torch.equal(snaps[:, t], pools[t]), "snapshot of token %d" % t
    assert torch.equal(pool_a, pool_b)


def test_verify_rollback():
    """Accept 2 of 5 drafts: restoring snapshot 1 and decoding on equals decoding only the
    2 accepted tokens and then the same continuation; without snapshots the pool ends as
    with them; one token equals one decode step."""
    import torch
    import linear_attention_recurrence_amd as gdn
    n_tok, accept = 5, 2
    d = workloads.make_decode(num_seqs=3, h_qk=1, h_v=2, ring=n_tok + 1, seed=141)
    dev, seq = _inputs(d, "bf16")
    pool_a = to_dev(d.pool)
    snaps = torch.empty((3, n_tok, 2, 128, 128), dtype=torch.float32, device="cuda")
    gdn.gdn_verify_step(seq["q"][:, :n_tok].contiguous(), seq["k"][:, :n_tok].contiguous(),
                        seq["v"][:, :n_tok].contiguous(), seq["g"][:, :n_tok].contiguous(),
                        seq["beta"][:, :n_tok].contiguous(), pool_a, d.scale, snapshots=snaps)
    pool_a.copy_(snaps[:, accept - 1])
    o_a = gdn.gdn_decode_step(dev["q"][n_tok], dev["k"][n_tok], dev["v"][n_tok], dev["g"][n_tok],
                              dev["beta"][n_tok], pool_a, d.scale)
    pool_b = to_dev(d.pool)
    gdn.gdn_verify_step(seq["q"][:, :accept].contiguous(), seq["k"][:, :accept].contiguous(),
                        seq["v"][:, :accept].contiguous(), seq["g"][:, :accept].contiguous(),
                        seq["beta"][:, :accept].contiguous(), pool_b, d.scale)
    o_b = gdn.gdn_decode_step(dev["q"][n_tok], dev["k"][n_tok], dev["v"][n_tok], dev["g"][n_tok],
                              dev["beta"][n_tok], pool_b, d.scale)
    pool_c = to_dev(d.pool)
    o1 = gdn.gdn_verify_step(seq["q"][:, :1].contiguous(), seq["k"][:, :1].contiguous(),
                             seq["v"][:, :1].contiguous(), seq["g"][:, :1].contiguous(),
                             seq["beta"][:, :1].contiguous(), pool_c, d.scale)
    pool_d = to_dev(d.pool)
    o2 = gdn.gdn_decode_step(dev["q"][0], dev["k"][0], dev["v"][0], dev["g"][0], dev["beta"][0],
                             pool_d, d.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(pool_a, pool_b)
    assert torch.equal(o1[:, 0], o2) and torch.equal(pool_c, pool_d)


def test_verify_model_size_against_oracle():
    """256 sequences x 4 drafts, 16 QK / 32 V heads, 512 MiB pool, snapshots (2 GiB): outputs,
    final states and snapshots of sampled (sequence, head) pairs against the fp64 recurrence."""
    import torch
    import linear_attention_recurrence_amd as gdn
    n_tok = 4
    d = workloads.make_decode(num_seqs=256, ring=n_tok, seed=142)
    _, seq = _inputs(d, "bf16")
    pool = to_dev(d.pool)
    snaps = torch.empty((256, n_tok, 32, 128, 128), dtype=torch.float32, device="cuda")
    o = gdn.gdn_verify_step(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"], pool, d.scale,
                            snapshots=snaps)
    torch.cuda.synchronize()
    f = workloads.bf16_bits_to_f32
    for n, h in ((0, 0), (17, 5), (128, 31), (255, 16)):
        j = h // 2
        q = f(d.q[:, n, j]).astype(np.float64)[:, None]
        k = f(d.k[:, n, j]).astype(np.float64)[:, None]
        v = f(d.v[:, n, h]).astype(np.float64)[:, None]
        g = d.g[:, n, h].astype(np.float64)[:, None]
        b = d.beta[:, n, h].astype(np.float64)[:, None]
        s0 = d.pool[n, h].astype(np.float64)
        o_ref, fin_ref, traj = oracle.recurrence(q, k, v, g, b, [0, n_tok], d.scale,
                                                 initial_state=s0[None, None], want_traj=True)
        check_outputs(to_host_f64(o[n, :, h]), o_ref[:, 0], "n%d h%d" % (n, h))
        check_state(to_host_f64(pool[n, h]), fin_ref[0, 0], "n%d h%d" % (n, h))
        for t in range(n_tok):
            check_state(to_host_f64(snaps[n, t, h]), traj[0, t], "n%d h%d snapshot %d" % (n, h, t))
