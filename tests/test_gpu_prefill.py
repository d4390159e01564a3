"""Prefill parity: libgdn's gdn_chunk_prefill against the fp64 oracle (GPU)."""

import numpy as np
import pytest

import workloads
from tests._util import (check_outputs, check_state, oracle_prefill, prefill_to_dev,
                         to_host_f64)

pytestmark = pytest.mark.gpu


def _run(x, with_final=True, alias=False):
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    N = x.num_seqs
    fin = None
    if alias:
        fin = d["s0"]
    elif with_final:
        fin = torch.full((N, x.h_v, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    o = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], x.scale,
                              initial_state=d["s0"], final_state=fin)
    torch.cuda.synchronize()
    return to_host_f64(o), (None if fin is None else to_host_f64(fin))


def _compare(x, o, fin, heads=None, seqs=None, label=""):
    ref = oracle_prefill(x, heads=heads, seqs=seqs)
    o_sel, r_sel, s_sel, rs_sel = [], [], [], []
    for (n, h), (o_ref, s_ref) in ref.items():
        t0, t1 = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        o_sel.append(o[t0:t1, h])
        r_sel.append(o_ref)
        if fin is not None:
            s_sel.append(fin[n, h])
            rs_sel.append(s_ref)
    res = check_outputs(np.concatenate(o_sel), np.concatenate(r_sel), label)
    if fin is not None:
        res = res + (check_state(np.stack(s_sel), np.stack(rs_sel), label),)
    print(label, "max|do| %.2e relF(o) %.2e" % res[:2], ("relF(S) %.2e" % res[2]) if len(res) > 2 else "")
    return res


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 128, 200])
@pytest.mark.parametrize("with_s0", [False, True])
def test_prefill_small_shapes(T, with_s0):
    x = workloads.make_prefill([T], h_qk=2, h_v=4, with_initial_state=with_s0, seed=100 + T)
    o, fin = _run(x)
    _compare(x, o, fin, label="T=%d s0=%s" % (T, with_s0))


def test_prefill_varlen_with_empty_sequences():
    lens = [0, 130, 0, 7, 64, 1, 191]
    x = workloads.make_prefill(lens, h_qk=2, h_v=4, with_initial_state=True, seed=7)
    o, fin = _run(x)
    _compare(x, o, fin, label="varlen")
    # empty sequences return their initial state unchanged
    for n in (0, 2):
        np.testing.assert_array_equal(fin[n], x.initial_state[n].astype(np.float64))


def test_prefill_varlen_equals_separate_calls():
    lens = [70, 3, 129]
    x = workloads.make_prefill(lens, h_qk=2, h_v=4, with_initial_state=True, seed=8)
    o, fin = _run(x)
    for n, L in enumerate(lens):
        t0 = int(x.cu_seqlens[n])
        sub = workloads.PrefillInputs(
            q=x.q[t0:t0 + L], k=x.k[t0:t0 + L], v=x.v[t0:t0 + L], g=x.g[t0:t0 + L],
            beta=x.beta[t0:t0 + L], cu_seqlens=np.array([0, L], dtype=np.int32),
            initial_state=x.initial_state[n:n + 1], scale=x.scale, io_dtype="bf16")
        o1, f1 = _run(sub)
        np.testing.assert_array_equal(o1, o[t0:t0 + L])
        np.testing.assert_array_equal(f1[0], fin[n])


def _sub_batch(x, first, last):
    """Sequences first..last-1 of a packed batch as a batch of their own."""
    t0, t1 = int(x.cu_seqlens[first]), int(x.cu_seqlens[last])
    return workloads.PrefillInputs(
        q=x.q[t0:t1], k=x.k[t0:t1], v=x.v[t0:t1], g=x.g[t0:t1], beta=x.beta[t0:t1],
        cu_seqlens=(x.cu_seqlens[first:last + 1] - t0).astype(np.int32),
        initial_state=x.initial_state[first:last], scale=x.scale, io_dtype="bf16")


def test_prefill_many_sequences_full_heads():
    """The state pass picks its workgroup shape from the number of (sequence, V head) pairs:
    12 sequences x 32 V heads take one workgroup of eight one-tile waves per head, which
    forms P^T on chip; 6 sequences take the same workgroup reading P^T from the workspace;
    4 sequences take two workgroups per head; 2 sequences and 1 take eight, with the chain
    on two waves and a read-out wave (two rounds of workgroups at 2 sequences), all reading
    P^T from the workspace. The per-row arithmetic, and P^T itself, are the same in all of
    them, so results must agree bit for bit."""
    lens = [0, 1, 64, 65, 200, 17, 128, 0, 311, 63, 90, 5]
    x = workloads.make_prefill(lens, h_qk=16, h_v=32, with_initial_state=True, seed=13)
    o, fin = _run(x)
    _compare(x, o, fin, label="12 seqs, 32 V heads")
    for first, last in ((2, 8), (4, 8), (8, 10), (4, 5), (8, 9)):
        ob, fb = _run(_sub_batch(x, first, last))
        t0, t1 = int(x.cu_seqlens[first]), int(x.cu_seqlens[last])
        np.testing.assert_array_equal(ob, o[t0:t1])
        np.testing.assert_array_equal(fb, fin[first:last])


@pytest.mark.parametrize("h_qk,h_v", [(1, 1), (4, 4), (2, 8), (1, 32)])
def test_prefill_head_groupings(h_qk, h_v):
    """V heads per QK head from 1 to 32 (the mapping h -> h / (h_v / h_qk))."""
    x = workloads.make_prefill([90, 0, 150], h_qk=h_qk, h_v=h_v, with_initial_state=True,
                               seed=20 + h_v)
    o, fin = _run(x)
    _compare(x, o, fin, label="h_qk=%d h_v=%d" % (h_qk, h_v))


@pytest.mark.parametrize("h_qk,h_v,n", [(1, 1, 33), (1, 1, 65), (1, 1, 129), (1, 1, 257),
                                         (1, 2, 17), (1, 2, 33), (1, 2, 65), (1, 2, 129)])
def test_prefill_shape_boundaries(h_qk, h_v, n):
    """(sequence, V head) pair counts just past each change of the state pass's workgroup
    shape (33, 65, 129 and 257 pairs, or 34, 66, 130 and 258), with 1 and 2 V heads per QK
    head, so the workgroup grids end in part-filled groups of eight QK heads: every head of
    sequences of 0 to 150 tokens against the oracle, with initial and final states."""
    rng = np.random.default_rng(1000 + 10 * h_v + n)
    lens = [int(v) for v in rng.integers(0, 151, n)]
    x = workloads.make_prefill(lens, h_qk=h_qk, h_v=h_v, with_initial_state=True, seed=2000 + n)
    o, fin = _run(x)
    _compare(x, o, fin, label="%d pairs" % (n * h_v))


def test_prefill_all_sequences_empty():
    """Zero tokens: every final state is its initial state, and nothing else is written."""
    x = workloads.make_prefill([0, 0, 0], h_qk=2, h_v=4, with_initial_state=True, seed=21)
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    fin = torch.full((3, 4, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    o = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], x.scale,
                              initial_state=d["s0"], final_state=fin)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    np.testing.assert_array_equal(to_host_f64(fin), x.initial_state.astype(np.float64))


def test_prefill_in_place_state_and_no_final():
    x = workloads.make_prefill([100, 37], h_qk=2, h_v=4, with_initial_state=True, seed=9)
    o_ref, fin_ref = _run(x)
    o2, fin2 = _run(x, alias=True)
    np.testing.assert_array_equal(o2, o_ref)
    np.testing.assert_array_equal(fin2, fin_ref)
    o3, _ = _run(x, with_final=False)
    np.testing.assert_array_equal(o3, o_ref)


def test_prefill_deterministic():
    x = workloads.make_prefill([333], h_qk=2, h_v=4, with_initial_state=True, seed=10)
    a = _run(x)
    b = _run(x)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_prefill_chaining_matches_whole():
    """prefill(T1) -> state -> prefill(T2) equals prefill(T1 + T2) (both on the GPU)."""
    T1, T2 = 100, 157
    x = workloads.make_prefill([T1 + T2], h_qk=2, h_v=4, with_initial_state=True, seed=11)
    o, fin = _run(x)
    sl = lambda a, s: a[s]
    p1 = workloads.PrefillInputs(q=x.q[:T1], k=x.k[:T1], v=x.v[:T1], g=x.g[:T1], beta=x.beta[:T1],
                                 cu_seqlens=np.array([0, T1], np.int32),
                                 initial_state=x.initial_state, scale=x.scale, io_dtype="bf16")
    o1, f1 = _run(p1)
    p2 = workloads.PrefillInputs(q=x.q[T1:], k=x.k[T1:], v=x.v[T1:], g=x.g[T1:], beta=x.beta[T1:],
                                 cu_seqlens=np.array([0, T2], np.int32),
                                 initial_state=f1.astype(np.float32), scale=x.scale, io_dtype="bf16")
    o2, f2 = _run(p2)
    check_outputs(np.concatenate([o1, o2]), o, "chain")
    check_state(f2, fin, "chain")


def test_config0_fp32():
    """B=1, T=256, 1 QK + 1 V head, fp32 I/O (token-sequential fp32 kernel)."""
    x = workloads.config0()
    o, fin = _run(x)
    res = _compare(x, o, fin, label="config0")
    assert res[1] < 1e-5 and res[2] < 1e-5     # fp32 end to end


def test_prefill_fp32_varlen():
    x = workloads.make_prefill([0, 5, 77], h_qk=2, h_v=4, io_dtype="f32", with_initial_state=True,
                               seed=12)
    o, fin = _run(x)
    res = _compare(x, o, fin, label="f32 varlen")
    assert res[1] < 1e-5 and res[2] < 1e-5


def test_prefill_fp32_many_pairs():
    """fp32 I/O with more than 64 (sequence, V head) pairs: the token-sequential kernel's
    other shape (8 rows per wave)."""
    x = workloads.make_prefill([0, 5, 77, 200], h_qk=8, h_v=32, io_dtype="f32",
                               with_initial_state=True, seed=14)
    o, fin = _run(x)
    res = _compare(x, o, fin, label="f32 128 pairs")
    assert res[1] < 1e-5 and res[2] < 1e-5


def test_config1_full():
    """B=1, T=4096, 16 QK / 32 V heads, bf16, S0 = 0: every head against the oracle."""
    x = workloads.config1()
    o, fin = _run(x)
    _compare(x, o, fin, label="config1")


def test_config2_all_heads():
    """B=1, T=32768, S0 ~ N(0, 0.02): the full launch, every V head against the oracle."""
    x = workloads.config2()
    o, fin = _run(x)
    _compare(x, o, fin, label="config2 all 32 heads")


def test_prefill_segmented_equals_other_shape():
    """With up to 32 (sequence, V head) pairs a call whose workspace would exceed one segment's
    runs in segments of 64 chunks per sequence (a prep and a state-pass launch each, the state
    between them in the workspace). One sequence of 9,000 tokens at 32 V heads (141 chunks,
    three segments) equals, bit for bit, the same sequence run inside a batch of three (96
    pairs: another state-pass shape, no segments), and the oracle on every head."""
    xb = workloads.make_prefill([9000, 70, 33], h_qk=16, h_v=32, with_initial_state=True, seed=41)
    ob, fb = _run(xb)
    x = _sub_batch(xb, 0, 1)
    o, fin = _run(x)
    np.testing.assert_array_equal(o, ob[:9000])
    np.testing.assert_array_equal(fin[0], fb[0])
    _compare(x, o, fin, label="segmented T=9000")


def test_prefill_segmented_two_rounds():
    """Segments with 64 pairs (two sequences at 32 V heads: the fewest-heads shape in two
    rounds of workgroups) of 9,000 and 5,000 tokens (141 and 79 chunks: three and two
    segments): equal, bit for bit, to the same sequences inside a batch of three (96 pairs:
    another shape, no segments), and the oracle on every head."""
    xb = workloads.make_prefill([9000, 5000, 33], h_qk=16, h_v=32, with_initial_state=True, seed=43)
    ob, fb = _run(xb)
    x = _sub_batch(xb, 0, 2)
    o, fin = _run(x)
    np.testing.assert_array_equal(o, ob[:14000])
    np.testing.assert_array_equal(fin, fb[:2])
    _compare(x, o, fin, label="segmented 64 pairs")


def test_prefill_segmented_many_small_heads():
    """Segments with 40 pairs (20 sequences of 3,000 to 6,000 tokens, 1 QK / 2 V heads: two
    rounds of workgroups, the last group of eight QK heads part-filled), sequences ending in
    different segments: every head against the oracle, and the same sequences in a batch
    with one more (the whole call at once, no segments) bit for bit."""
    rng = np.random.default_rng(44)
    lens = [int(v) for v in rng.integers(3000, 6001, 20)]
    x = workloads.make_prefill(lens + [33] * 13, h_qk=1, h_v=2, with_initial_state=True, seed=45)
    ob, fb = _run(x)            # 66 pairs: no segments
    xs = _sub_batch(x, 0, 20)   # 40 pairs: segments
    o, fin = _run(xs)
    np.testing.assert_array_equal(o, ob[:xs.total_tokens])
    np.testing.assert_array_equal(fin, fb[:20])
    _compare(xs, o, fin, label="segmented 40 pairs")


def test_prefill_segmented_varlen():
    """Segments over several sequences (4 QK / 8 V heads: three sequences are 24 pairs) of
    4200, 0 and 12000 tokens (66, 0 and 188 chunks): the first ends in the second segment,
    the empty one returns its initial state, the third runs three segments and the fourth
    has no work. Against the oracle; the state written over the initial one in place and
    a call without a final state give the same outputs."""
    x = workloads.make_prefill([4200, 0, 12000], h_qk=4, h_v=8, with_initial_state=True, seed=42)
    o, fin = _run(x)
    _compare(x, o, fin, label="segmented varlen")
    np.testing.assert_array_equal(fin[1], x.initial_state[1].astype(np.float64))
    o2, fin2 = _run(x, alias=True)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(fin2, fin)
    o3, _ = _run(x, with_final=False)
    np.testing.assert_array_equal(o3, o)


def test_prefill_on_side_stream_equals_current_stream():
    """A call launched on a stream other than torch's current one, with the binding
    allocating o and the workspace: the allocations belong to that stream, so work queued
    on the current stream right after cannot be handed their memory while the call runs.
    Results equal those of the same call on the current stream, bit for bit."""
    import torch
    import linear_attention_recurrence_amd as gdn
    x = workloads.make_prefill([300, 77], h_qk=16, h_v=32, with_initial_state=True, seed=31)
    d = prefill_to_dev(x)
    o_ref = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], x.scale,
                                  initial_state=d["s0"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                          x.scale, initial_state=d["s0"], stream=side))
        # allocations and writes on the current stream while the side-stream call runs
        junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda").fill_(0xFF)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(to_host_f64(o), to_host_f64(o_ref))
