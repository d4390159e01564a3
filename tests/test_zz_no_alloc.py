"""gdn_chunk_prefill_noalloc (the prefill whose workspace is the library's own device scratch)
against gdn_chunk_prefill, through the C ABI (GPU).

Two calls in a row on the scratch -- the second smaller, so it runs over what the first left
there -- each equal bit for bit to gdn_chunk_prefill with a caller workspace (the same
kernels), and the first within the parity bars of the fp64 oracle; a long sequence, which
runs in segments; a batch that fits only in segments, in two rounds of workgroups; a size
beyond the scratch is rejected with nothing written.
"""

import numpy as np
import pytest

import workloads
from tests._util import check_outputs, check_state, oracle_prefill, prefill_to_dev, to_host_f64

pytestmark = pytest.mark.gpu

GDN_ERR_WORKSPACE = 4


def _both(x):
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    N, T = x.num_seqs, x.total_tokens
    outs = []
    for fn in ("gdn_chunk_prefill", "gdn_chunk_prefill_noalloc"):
        o = torch.full((T, x.h_v, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        fin = torch.full((N, x.h_v, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        if fn == "gdn_chunk_prefill":
            gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], x.scale,
                                  initial_state=d["s0"], final_state=fin, o=o)
        else:
            gdn.gdn_chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                          x.scale, o, initial_state=d["s0"], final_state=fin)
        torch.cuda.synchronize()
        outs.append((to_host_f64(o), to_host_f64(fin)))
    return outs


def test_noalloc_equals_prefill_two_calls():
    # first call: one sequence of 5,000 tokens, 32 V heads (two segments)
    x1 = workloads.make_prefill([5000], with_initial_state=True, seed=901)
    (o_ref, f_ref), (o_na, f_na) = _both(x1)
    np.testing.assert_array_equal(o_na, o_ref)
    np.testing.assert_array_equal(f_na, f_ref)
    ref = oracle_prefill(x1)
    check_outputs(np.stack([o_na[:, h] for h in range(32)]), np.stack([ref[(0, h)][0] for h in range(32)]),
                  "noalloc T=5000")
    check_state(f_na[0], np.stack([ref[(0, h)][1] for h in range(32)]), "noalloc T=5000")
    # second call, smaller: a ragged batch of two sequences over what the first call left
    x2 = workloads.make_prefill([300, 77], with_initial_state=True, seed=902)
    (o_ref2, f_ref2), (o_na2, f_na2) = _both(x2)
    np.testing.assert_array_equal(o_na2, o_ref2)
    np.testing.assert_array_equal(f_na2, f_ref2)


def test_noalloc_long_sequence_in_segments():
    """One sequence of 32,768 tokens at 32 V heads runs in segments whose workspace fits the
    scratch: equal bit for bit to gdn_chunk_prefill."""
    x = workloads.make_prefill([32768], with_initial_state=True, seed=904)
    (o_ref, f_ref), (o_na, f_na) = _both(x)
    np.testing.assert_array_equal(o_na, o_ref)
    np.testing.assert_array_equal(f_na, f_ref)


def test_noalloc_segments_in_two_rounds():
    """35 sequences of 5,000 tokens at 1 QK / 1 V head (35 pairs: two rounds of state-pass
    workgroups): the whole call's blocks (70.9 MB) would exceed the scratch, the segments'
    (59.6 MB) fit, so the call runs in segments; equal bit for bit to gdn_chunk_prefill."""
    x = workloads.make_prefill([5000] * 35, h_qk=1, h_v=1, with_initial_state=True, seed=905)
    (o_ref, f_ref), (o_na, f_na) = _both(x)
    np.testing.assert_array_equal(o_na, o_ref)
    np.testing.assert_array_equal(f_na, f_ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """Two sequences at 32 V heads (64 pairs) of 2,600 tokens each need 84 blocks of 32 x
    25,600 bytes (fewer than two segments' 104 MiB, so no segments), more than the 64 MiB
    scratch."""
    import torch
    import linear_attention_recurrence_amd as gdn
    x = workloads.make_prefill([2600, 2600], h_qk=16, h_v=32, seed=903)
    d = prefill_to_dev(x)
    o = torch.full((5200, 32, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                      x.scale, o)
    assert e.value.status == GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
