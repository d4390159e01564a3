"""Decode parity: gdn_decode_step against the fp64 oracle and against prefill (GPU)."""

import numpy as np
import pytest

import oracle
import workloads
from tests._util import check_outputs, check_state, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _oracle_chain(d, slot, n, h, steps, state0):
    """fp64 oracle of one (sequence n, V head h) over the given decode steps."""
    R = d.q.shape[0]
    group = d.v.shape[2] // d.q.shape[2]
    idx = [s % R for s in steps]
    j = h // group
    f = workloads.bf16_bits_to_f32
    q = f(d.q[idx, n, j]).astype(np.float64)[:, None]
    k = f(d.k[idx, n, j]).astype(np.float64)[:, None]
    v = f(d.v[idx, n, h]).astype(np.float64)[:, None]
    g = d.g[idx, n, h].astype(np.float64)[:, None]
    b = d.beta[idx, n, h].astype(np.float64)[:, None]
    o, fin, _ = oracle.recurrence(q, k, v, g, b, [0, len(idx)], d.scale,
                                  initial_state=state0[None, None])
    return o[:, 0], fin[0, 0]


def _step(d, dev, r, o=None):
    import linear_attention_recurrence_amd as gdn
    return gdn.gdn_decode_step(dev["q"][r], dev["k"][r], dev["v"][r], dev["g"][r], dev["beta"][r],
                               dev["pool"], d.scale, state_slots=dev["slots"], o=o)


def _dev(d):
    return dict(q=to_dev(d.q), k=to_dev(d.k), v=to_dev(d.v), g=to_dev(d.g), beta=to_dev(d.beta),
                pool=to_dev(d.pool), slots=to_dev(d.slots))


@pytest.mark.parametrize("permuted", [False, True])
def test_decode_small_many_steps(permuted):
    import torch
    d = workloads.make_decode(num_seqs=5, h_qk=2, h_v=4, ring=3, pool_size=9 if permuted else None,
                              permuted_slots=permuted, seed=40)
    dev = _dev(d)
    pool0 = d.pool.astype(np.float64)
    steps = 20
    outs = []
    for s in range(steps):
        outs.append(to_host_f64(_step(d, dev, s % 3)))
    torch.cuda.synchronize()
    pool = to_host_f64(dev["pool"])
    for n in range(5):
        slot = int(d.slots[n]) if permuted else n
        for h in range(4):
            o_ref, s_ref = _oracle_chain(d, slot, n, h, list(range(steps)), pool0[slot, h])
            check_outputs(np.stack([o[n, h] for o in outs]), o_ref, "n%d h%d" % (n, h))
            check_state(pool[slot, h], s_ref, "n%d h%d" % (n, h))
    if permuted:   # untouched pool entries stay bit-identical
        unused = sorted(set(range(9)) - set(int(s) for s in d.slots))
        np.testing.assert_array_equal(pool[unused], pool0[unused])


def test_config3_one_step_full():
    """256 sequences x 32 V heads, fp32 pool of 512 MiB: the whole step against the oracle."""
    import torch
    d = workloads.config3()
    dev = _dev(d)
    o = to_host_f64(_step(d, dev, 0))
    torch.cuda.synchronize()
    pool = to_host_f64(dev["pool"])
    f = workloads.bf16_bits_to_f32
    N = 256
    q = f(d.q[0]).astype(np.float64)             # [N][16][128]
    k = f(d.k[0]).astype(np.float64)
    # a packed batch of N sequences of one token each
    o_ref, fin_ref, _ = oracle.recurrence(q, k, f(d.v[0]).astype(np.float64),
                                          d.g[0].astype(np.float64), d.beta[0].astype(np.float64),
                                          np.arange(N + 1), d.scale,
                                          initial_state=d.pool.astype(np.float64))
    check_outputs(o, o_ref, "config3 step 1")
    check_state(pool, fin_ref, "config3 step 1")


def _oracle_chains(d, chains, steps, pool0):
    """fp64 oracle of many (sequence n, V head h) chains over the same decode steps, as one
    packed batch (one single-head sequence per chain) so the oracle's threads share it."""
    R = d.q.shape[0]
    group = d.v.shape[2] // d.q.shape[2]
    idx = np.array([s % R for s in steps])
    f = workloads.bf16_bits_to_f32
    L = len(idx)
    q = np.concatenate([f(d.q[idx, n, h // group]) for n, h in chains]).astype(np.float64)[:, None]
    k = np.concatenate([f(d.k[idx, n, h // group]) for n, h in chains]).astype(np.float64)[:, None]
    v = np.concatenate([f(d.v[idx, n, h]) for n, h in chains]).astype(np.float64)[:, None]
    g = np.concatenate([d.g[idx, n, h] for n, h in chains]).astype(np.float64)[:, None]
    b = np.concatenate([d.beta[idx, n, h] for n, h in chains]).astype(np.float64)[:, None]
    s0 = np.stack([pool0[n, h] for n, h in chains])[:, None]
    cu = np.arange(len(chains) + 1) * L
    o, fin, _ = oracle.recurrence(q, k, v, g, b, cu, d.scale, initial_state=s0)
    return o[:, 0].reshape(len(chains), L, -1), fin[:, 0]


def test_config3_thousand_steps():
    """1000 consecutive steps over the ring of 16 input sets. One chain of every sequence
    (512 chains: every sequence twice, its V head cycling through all 32) is checked at
    steps 1 and 1000 and in the pool after the last step; the whole first step is checked
    by test_config3_one_step_full."""
    import torch
    d = workloads.config3()
    dev = _dev(d)
    pool0 = d.pool.astype(np.float64)
    o_first = to_host_f64(_step(d, dev, 0))
    o_buf = torch.empty_like(dev["v"][0])
    for s in range(1, 1000):
        _step(d, dev, s % 16, o=o_buf)
    torch.cuda.synchronize()
    o_last = to_host_f64(o_buf)
    pool = to_host_f64(dev["pool"])
    chains = [(n, (n + 13 * r) % 32) for r in range(2) for n in range(256)]
    o_ref, s_ref = _oracle_chains(d, chains, list(range(1000)), pool0)
    idx_n = np.array([c[0] for c in chains])
    idx_h = np.array([c[1] for c in chains])
    check_outputs(o_first[idx_n, idx_h], o_ref[:, 0], "step 1")
    check_outputs(o_last[idx_n, idx_h], o_ref[:, -1], "step 1000")
    check_state(pool[idx_n, idx_h], s_ref, "pool after step 1000")


def test_prefill_equals_decode_steps():
    """T decode steps of one sequence equal a prefill over the same T tokens (GPU only)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    T = 70
    x = workloads.make_prefill([T], h_qk=2, h_v=4, with_initial_state=True, seed=44)
    qd, kd, vd = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    gd, bd = to_dev(x.g), to_dev(x.beta)
    s0 = to_dev(x.initial_state)
    fin = torch.empty_like(s0)
    o_pf = gdn.gdn_chunk_prefill(qd, kd, vd, gd, bd, to_dev(x.cu_seqlens), x.scale,
                                 initial_state=s0, final_state=fin)
    pool = s0.clone()
    outs = []
    for t in range(T):
        outs.append(gdn.gdn_decode_step(qd[t:t + 1], kd[t:t + 1], vd[t:t + 1], gd[t:t + 1],
                                        bd[t:t + 1], pool, x.scale))
    torch.cuda.synchronize()
    o_dec = torch.cat(outs)
    check_outputs(to_host_f64(o_pf), to_host_f64(o_dec), "prefill vs decode")
    check_state(to_host_f64(fin), to_host_f64(pool), "prefill vs decode")
