"""Chunked-prefill parity against the fp64 oracle where the chunked form is fragile (GPU).

The decay alpha and the write strength beta of the update (page "Qwen3-Next -- How a running
memory and a searchable history cooperate", section "Correcting a memory instead of adding
to it") are taken to their limits: alpha = 1; alpha = e^-5 per token, so the running decay
underflows inside a 64-token chunk; beta = 0.999 with one key repeated over a whole chunk,
or with two nearly parallel keys alternating (the unit-lower-triangular system of a chunk
is then at its worst); and all-zero key and query rows in mid-chunk. Each runs at lengths
64, 65 and 200 (a whole chunk, a one-token tail, several chunks with a ragged tail), with
and without an initial state, and through every workgroup shape of the state pass, which
the library picks from the number of (sequence, V head) pairs: 32 pairs (eight workgroups
per head with the chain on two waves and a read-out wave), 64 (the same in two rounds of
workgroups), 128 (two workgroups per head), 160 (one workgroup of eight waves per head) and
288 (the same, forming P^T on chip). The same tolerances as every other prefill test.
"""

import numpy as np
import pytest

import workloads
from tests._util import check_outputs, check_state, oracle_prefill, prefill_to_dev, to_host_f64

pytestmark = pytest.mark.gpu

# number of sequences of the 16 QK / 32 V head shape -> the state pass's workgroup shape
SHAPES = {"ro_32pairs": 1, "ro_64pairs": 2, "wg2_128pairs": 4, "wg1_160pairs": 5, "form_288pairs": 9}


def _run(x):
    import torch
    import linear_attention_recurrence_amd as gdn
    d = prefill_to_dev(x)
    fin = torch.full((x.num_seqs, x.h_v, 128, 128), float("nan"), dtype=torch.float32,
                     device="cuda")
    o = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], x.scale,
                              initial_state=d["s0"], final_state=fin)
    torch.cuda.synchronize()
    return to_host_f64(o), to_host_f64(fin)


def _check(x, o, fin, label):
    ref = oracle_prefill(x)
    o_sel, r_sel, s_sel, rs_sel = [], [], [], []
    for (n, h), (o_ref, s_ref) in ref.items():
        t0, t1 = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        o_sel.append(o[t0:t1, h])
        r_sel.append(o_ref)
        s_sel.append(fin[n, h])
        rs_sel.append(s_ref)
    assert np.isfinite(o).all() and np.isfinite(fin).all(), label
    ma, rf = check_outputs(np.concatenate(o_sel), np.concatenate(r_sel), label)
    rs = check_state(np.stack(s_sel), np.stack(rs_sel), label)
    print(label, "max|do| %.2e relF(o) %.2e relF(S) %.2e" % (ma, rf, rs))


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("T", [64, 65, 200])
@pytest.mark.parametrize("case", workloads.EDGE_CASES)
def test_chunked_prefill_edge(case, T, with_s0, shape):
    n = SHAPES[shape]
    x = workloads.make_prefill_edge(case, [T] * n, with_initial_state=with_s0,
                                    seed=300 + T + 7 * n + (1000 if with_s0 else 0))
    o, fin = _run(x)
    _check(x, o, fin, "%s T=%d s0=%s %s" % (case, T, with_s0, shape))


@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("case", workloads.EDGE_CASES)
def test_fp32_prefill_edge(case, T):
    """The same regimes through the fp32-I/O prefill (token-sequential fp32 kernel), with
    full-precision fp32 inputs and the fp32 path's own bound."""
    x = workloads.make_prefill_edge(case, [T, 3], h_qk=2, h_v=4, io_dtype="f32",
                                    with_initial_state=True, seed=500 + T)
    o, fin = _run(x)
    ref = oracle_prefill(x)
    o_sel = np.concatenate([o[int(x.cu_seqlens[n]):int(x.cu_seqlens[n + 1]), h] for (n, h) in ref])
    r_sel = np.concatenate([r[0] for r in ref.values()])
    s_sel = np.stack([fin[n, h] for (n, h) in ref])
    rs_sel = np.stack([r[1] for r in ref.values()])
    ma, rf = check_outputs(o_sel, r_sel, case)
    rs = check_state(s_sel, rs_sel, case)
    assert rf < 1e-5 and rs < 1e-5, "%s relF(o) %.2e relF(S) %.2e" % (case, rf, rs)
