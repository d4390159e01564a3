"""The C ABI on the CPU: libgdn.so loads, exports what include/gdn.h declares, and rejects
bad arguments on the host before any launch (no GPU needed: validation happens first)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from linear_attention_recurrence_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return L.load(), L


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(["gdn_status_string", "gdn_chunk_prefill_workspace_bytes",
                                            "gdn_chunk_prefill", "gdn_decode_step", "gdn_verify_step",
                                            "gdn_channel_decay_prefill",
                                            "gdn_channel_decay_decode_step",
                                            "gdn_conv_prep", "gdn_conv_decode_step",
                                            "gdn_conv_window_from_prefill", "gdn_gated_rmsnorm",
                                            "gdn_decode_step_with_conv",
                                            "gdn_chunk_prefill_noalloc",
                                            "gdn_chunk_prefill_conv_workspace_bytes",
                                            "gdn_chunk_prefill_conv"])


def test_library_exports_every_declared_symbol():
    lib, L = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(L.EXPORTED) == set(_declared_functions())


def test_status_strings():
    lib, L = _lib()
    for s in range(6):
        assert lib.gdn_status_string(s).decode().startswith("GDN_")
    assert lib.gdn_status_string(99) == b"unknown gdn_status"


def test_workspace_query():
    """The documented size: per chunk 25600 B per V head, for ceil(T / 64) + N chunks; with at
    most 64 (sequence, V head) pairs, the segmented size N (64 h_v 25600 + h_v 128^2 4) when
    that is smaller, independent of T; none (0) with no tokens."""
    lib, _ = _lib()
    for T, N, h_qk, h_v in ((4096, 1, 16, 32), (32768, 1, 16, 32), (10 ** 6, 1, 16, 32), (276989, 64, 16, 32),
                            (0, 3, 16, 32), (65, 2, 16, 32), (4224, 1, 16, 32), (4160, 1, 16, 32),
                            (16200, 3, 4, 8), (5000, 4, 4, 8), (20000, 2, 16, 32), (20000, 3, 16, 32),
                            (60000, 8, 4, 8), (60000, 9, 4, 8)):
        whole = (-(-T // 64) + N) * h_v * 25600
        seg = N * (64 * h_v * 25600 + h_v * 128 * 128 * 4)
        expect = seg if N * h_v <= 64 and seg < whole else whole
        if T == 0:
            expect = 0   # no chunks: the call only copies initial to final states
        assert lib.gdn_chunk_prefill_workspace_bytes(T, N, h_qk, h_v, 128, 128) == expect
    assert lib.gdn_chunk_prefill_workspace_bytes(32768, 1, 16, 32, 128, 128) == 54_525_952
    assert lib.gdn_chunk_prefill_workspace_bytes(4096, 1, 16, 32, 128, 128) == 65 * 32 * 25600
    assert lib.gdn_chunk_prefill_workspace_bytes(-1, 1, 16, 32, 128, 128) == 0
    assert lib.gdn_chunk_prefill_workspace_bytes(10, 1, 16, 30, 128, 128) == 0
    assert lib.gdn_chunk_prefill_workspace_bytes(10, 1, 16, 32, 64, 128) == 0


def _fake(n=1):
    # addresses are never dereferenced: every call below fails validation first
    return ctypes.c_void_p(0x1000 * n)


def test_decode_validation():
    lib, L = _lib()
    f = lib.gdn_decode_step
    P = _fake
    ok = dict(q=P(1), k=P(2), v=P(3), dt=L.GDN_BF16, g=P(4), b=P(5), pool=P(6), slots=None,
              n=4, hqk=16, hv=32, dk=128, dv=128, sc=1.0, o=P(7), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["dt"], a["g"], a["b"], a["pool"], a["slots"], a["n"],
                 a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["o"], a["st"])

    assert call(q=None) == L.GDN_ERR_NULL
    assert call(pool=None) == L.GDN_ERR_NULL
    assert call(o=None) == L.GDN_ERR_NULL
    assert call(n=-1) == L.GDN_ERR_SHAPE
    assert call(hv=30) == L.GDN_ERR_SHAPE
    assert call(hqk=0) == L.GDN_ERR_SHAPE
    assert call(dk=64) == L.GDN_ERR_UNSUPPORTED
    assert call(dv=256) == L.GDN_ERR_UNSUPPORTED
    assert call(dt=7) == L.GDN_ERR_UNSUPPORTED
    assert call(n=0, q=None, pool=None) == L.GDN_OK     # nothing to do, nothing launched


def test_prefill_validation():
    lib, L = _lib()
    f = lib.gdn_chunk_prefill
    P = _fake
    ok = dict(q=P(1), k=P(2), v=P(3), dt=L.GDN_BF16, g=P(4), b=P(5), cu=P(6), n=2, T=100,
              hqk=16, hv=32, dk=128, dv=128, sc=0.1, s0=None, sf=None, o=P(7), ws=None, wsb=0,
              st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["dt"], a["g"], a["b"], a["cu"], a["n"], a["T"],
                 a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["s0"], a["sf"], a["o"], a["ws"],
                 a["wsb"], a["st"])

    assert call(cu=None) == L.GDN_ERR_NULL
    assert call(k=None) == L.GDN_ERR_NULL
    assert call(b=None) == L.GDN_ERR_NULL
    assert call(T=-5) == L.GDN_ERR_SHAPE
    assert call(n=-1) == L.GDN_ERR_SHAPE
    assert call(n=0, T=10) == L.GDN_ERR_SHAPE
    assert call(hqk=3, hv=32) == L.GDN_ERR_SHAPE
    assert call(dk=96) == L.GDN_ERR_UNSUPPORTED
    assert call(dt=2) == L.GDN_ERR_UNSUPPORTED
    assert call(ws=None) == L.GDN_ERR_WORKSPACE
    assert call(ws=P(8), wsb=1000) == L.GDN_ERR_WORKSPACE
    assert call(n=0, T=0) == L.GDN_OK


def test_prefill_noalloc_validation():
    """The variant that allocates nothing validates like gdn_chunk_prefill and rejects, with
    nothing launched, sizes whose workspace would exceed its device scratch."""
    lib, L = _lib()
    f = lib.gdn_chunk_prefill_noalloc
    P = _fake
    ok = dict(q=P(1), k=P(2), v=P(3), dt=L.GDN_BF16, g=P(4), b=P(5), cu=P(6), n=1, T=100,
              hqk=16, hv=32, dk=128, dv=128, sc=0.1, s0=None, sf=None, o=P(7), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["dt"], a["g"], a["b"], a["cu"], a["n"], a["T"],
                 a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["s0"], a["sf"], a["o"], a["st"])

    assert call(cu=None) == L.GDN_ERR_NULL
    assert call(o=None) == L.GDN_ERR_NULL
    assert call(T=-5) == L.GDN_ERR_SHAPE
    assert call(n=0, T=10) == L.GDN_ERR_SHAPE
    assert call(hqk=3, hv=32) == L.GDN_ERR_SHAPE
    assert call(dk=96) == L.GDN_ERR_UNSUPPORTED
    assert call(dt=2) == L.GDN_ERR_UNSUPPORTED
    assert call(n=0, T=0) == L.GDN_OK
    # the scratch limit: one sequence at 32 V heads runs in segments whatever its length;
    # two sequences (64 pairs) hold the whole call's blocks while those are fewer than two
    # segments' (104 MiB), and fit up to ceil(T / 64) + 2 = 81 chunks
    need = lambda T, n: L.gdn_chunk_prefill_workspace_bytes(T, n, 16, 32, 128, 128)
    assert need(10 ** 7, 1) <= L.NOALLOC_SCRATCH_BYTES
    assert need(5056, 2) <= L.NOALLOC_SCRATCH_BYTES < need(5057, 2)
    assert call(T=5057, n=2) == L.GDN_ERR_WORKSPACE
    assert call(T=200, n=80) == L.GDN_ERR_WORKSPACE       # ceil(200 / 64) + 80 > 81 chunks


def test_prefill_conv_validation():
    """The prefill with the front end validates like gdn_chunk_prefill and gdn_conv_prep, and
    its workspace query adds the q, k, v pass only where the front end does not run inside."""
    lib, L = _lib()
    f = lib.gdn_chunk_prefill_conv
    P = _fake
    ok = dict(x=P(1), w=P(2), K=4, qs=0.1, g=P(4), b=P(5), cu=P(6), n=64, T=1000, hqk=16, hv=32,
              dk=128, dv=128, sc=1.0, s0=None, sf=None, o=P(7), ws=None, wsb=0, st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["K"], a["qs"], a["g"], a["b"], a["cu"], a["n"], a["T"], a["hqk"],
                 a["hv"], a["dk"], a["dv"], a["sc"], a["s0"], a["sf"], a["o"], a["ws"], a["wsb"], a["st"])

    assert call(x=None) == L.GDN_ERR_NULL
    assert call(w=None) == L.GDN_ERR_NULL
    assert call(cu=None) == L.GDN_ERR_NULL
    assert call(K=0) == L.GDN_ERR_SHAPE
    assert call(K=5) == L.GDN_ERR_UNSUPPORTED
    assert call(T=-1) == L.GDN_ERR_SHAPE
    assert call(dk=64) == L.GDN_ERR_UNSUPPORTED
    assert call() == L.GDN_ERR_WORKSPACE
    assert call(ws=P(8), wsb=100) == L.GDN_ERR_WORKSPACE
    assert call(n=0, T=0) == L.GDN_OK
    q = lambda T, n: lib.gdn_chunk_prefill_conv_workspace_bytes(T, n, 16, 32, 128, 128)
    p = lambda T, n: lib.gdn_chunk_prefill_workspace_bytes(T, n, 16, 32, 128, 128)
    assert q(276989, 64) == p(276989, 64) + 276989 * 8192 * 2   # q, k and v after the blocks
    assert q(4096, 1) == p(4096, 1) + 4096 * 8192 * 2
    assert q(-1, 1) == 0
    assert q(0, 3) == 0 and p(0, 3) == 0


def test_conv_prep_validation():
    lib, L = _lib()
    f = lib.gdn_conv_prep
    P = _fake
    ok = dict(x=P(1), w=P(2), K=4, cu=P(3), n=2, T=10, hqk=16, hv=32, dk=128, dv=128, qs=0.1,
              q=P(4), k=P(5), v=P(6), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["K"], a["cu"], a["n"], a["T"], a["hqk"], a["hv"], a["dk"],
                 a["dv"], a["qs"], a["q"], a["k"], a["v"], a["st"])

    assert call(x=None) == L.GDN_ERR_NULL
    assert call(w=None) == L.GDN_ERR_NULL
    assert call(v=None) == L.GDN_ERR_NULL
    assert call(K=0) == L.GDN_ERR_SHAPE
    assert call(K=5) == L.GDN_ERR_UNSUPPORTED
    assert call(dv=64) == L.GDN_ERR_UNSUPPORTED
    assert call(T=-1) == L.GDN_ERR_SHAPE
    assert call(T=0) == L.GDN_OK


def test_verify_validation():
    lib, L = _lib()
    f = lib.gdn_verify_step
    P = _fake
    ok = dict(q=P(1), k=P(2), v=P(3), dt=0, g=P(4), b=P(5), pool=P(6), slots=None, snap=None,
              n=2, nt=3, hqk=16, hv=32, dk=128, dv=128, sc=0.1, o=P(7), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["dt"], a["g"], a["b"], a["pool"], a["slots"],
                 a["snap"], a["n"], a["nt"], a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["o"],
                 a["st"])

    assert call(q=None) == L.GDN_ERR_NULL
    assert call(b=None) == L.GDN_ERR_NULL
    assert call(pool=None) == L.GDN_ERR_NULL
    assert call(o=None) == L.GDN_ERR_NULL
    assert call(n=-1) == L.GDN_ERR_SHAPE
    assert call(nt=-1) == L.GDN_ERR_SHAPE
    assert call(hv=24) == L.GDN_ERR_SHAPE
    assert call(dk=64) == L.GDN_ERR_UNSUPPORTED
    assert call(dt=7) == L.GDN_ERR_UNSUPPORTED
    assert call(nt=0) == L.GDN_OK
    assert call(n=0) == L.GDN_OK


def test_channel_decay_validation():
    lib, L = _lib()
    P = _fake
    f = lib.gdn_channel_decay_prefill
    ok = dict(q=P(1), k=P(2), v=P(3), dt=0, g=P(4), b=P(5), cu=P(6), n=2, T=10, hqk=16, hv=32,
              dk=128, dv=128, sc=0.1, s0=None, sf=None, o=P(7), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["dt"], a["g"], a["b"], a["cu"], a["n"], a["T"],
                 a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["s0"], a["sf"], a["o"], a["st"])

    assert call(g=None) == L.GDN_ERR_NULL
    assert call(cu=None) == L.GDN_ERR_NULL
    assert call(T=-1) == L.GDN_ERR_SHAPE
    assert call(n=0) == L.GDN_ERR_SHAPE
    assert call(dt=3) == L.GDN_ERR_UNSUPPORTED
    assert call(dv=64) == L.GDN_ERR_UNSUPPORTED
    assert call(T=0) == L.GDN_OK
    d = lib.gdn_channel_decay_decode_step
    assert d(P(1), P(2), P(3), 0, None, P(5), P(6), None, 2, 16, 32, 128, 128, 0.1, P(7), None) == L.GDN_ERR_NULL
    assert d(P(1), P(2), P(3), 0, P(4), P(5), None, None, 2, 16, 32, 128, 128, 0.1, P(7), None) == L.GDN_ERR_NULL
    assert d(P(1), P(2), P(3), 0, P(4), P(5), P(6), None, -1, 16, 32, 128, 128, 0.1, P(7), None) == L.GDN_ERR_SHAPE
    assert d(P(1), P(2), P(3), 0, P(4), P(5), P(6), None, 0, 16, 32, 128, 128, 0.1, P(7), None) == L.GDN_OK


def test_conv_decode_validation():
    lib, L = _lib()
    f = lib.gdn_conv_decode_step
    P = _fake
    ok = dict(x=P(1), w=P(2), K=4, win=P(3), slots=None, n=2, hqk=16, hv=32, dk=128, dv=128,
              qs=0.1, q=P(4), k=P(5), v=P(6), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["K"], a["win"], a["slots"], a["n"], a["hqk"], a["hv"], a["dk"],
                 a["dv"], a["qs"], a["q"], a["k"], a["v"], a["st"])

    assert call(x=None) == L.GDN_ERR_NULL
    assert call(w=None) == L.GDN_ERR_NULL
    assert call(win=None) == L.GDN_ERR_NULL
    assert call(q=None) == L.GDN_ERR_NULL
    assert call(K=0) == L.GDN_ERR_SHAPE
    assert call(K=5) == L.GDN_ERR_UNSUPPORTED
    assert call(n=-1) == L.GDN_ERR_SHAPE
    assert call(hv=30) == L.GDN_ERR_SHAPE
    assert call(dk=64) == L.GDN_ERR_UNSUPPORTED
    assert call(n=0) == L.GDN_OK


def test_conv_window_validation():
    lib, L = _lib()
    f = lib.gdn_conv_window_from_prefill
    P = _fake
    ok = dict(x=P(1), K=4, cu=P(2), n=2, T=10, hqk=16, hv=32, dk=128, dv=128, win=P(3),
              slots=None, st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["K"], a["cu"], a["n"], a["T"], a["hqk"], a["hv"], a["dk"], a["dv"],
                 a["win"], a["slots"], a["st"])

    assert call(x=None) == L.GDN_ERR_NULL
    assert call(cu=None) == L.GDN_ERR_NULL
    assert call(win=None) == L.GDN_ERR_NULL
    assert call(K=0) == L.GDN_ERR_SHAPE
    assert call(K=5) == L.GDN_ERR_UNSUPPORTED
    assert call(T=-1) == L.GDN_ERR_SHAPE
    assert call(n=0) == L.GDN_ERR_SHAPE
    assert call(n=0, T=0) == L.GDN_OK
    assert call(K=1, win=None) == L.GDN_OK


def test_gated_rmsnorm_validation():
    lib, L = _lib()
    f = lib.gdn_gated_rmsnorm
    P = _fake
    ok = dict(o=P(1), z=P(2), dt=L.GDN_BF16, w=P(3), rows=10, hv=32, dv=128, eps=1e-6, gate=0,
              out=P(4), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["o"], a["z"], a["dt"], a["w"], a["rows"], a["hv"], a["dv"], a["eps"],
                 a["gate"], a["out"], a["st"])

    assert call(o=None) == L.GDN_ERR_NULL
    assert call(z=None) == L.GDN_ERR_NULL
    assert call(w=None) == L.GDN_ERR_NULL
    assert call(out=None) == L.GDN_ERR_NULL
    assert call(rows=-1) == L.GDN_ERR_SHAPE
    assert call(hv=0) == L.GDN_ERR_SHAPE
    assert call(eps=-1.0) == L.GDN_ERR_SHAPE
    assert call(eps=float("nan")) == L.GDN_ERR_SHAPE
    assert call(eps=float("inf")) == L.GDN_ERR_SHAPE
    assert call(dv=64) == L.GDN_ERR_UNSUPPORTED
    assert call(dt=7) == L.GDN_ERR_UNSUPPORTED
    assert call(gate=2) == L.GDN_ERR_UNSUPPORTED
    assert call(rows=2 ** 31 - 1, hv=2 ** 20) == L.GDN_ERR_UNSUPPORTED
    assert call(rows=0) == L.GDN_OK
    assert call(rows=0, o=None, z=None, w=None, out=None) == L.GDN_OK


def test_decode_with_conv_validation():
    lib, L = _lib()
    f = lib.gdn_decode_step_with_conv
    P = _fake
    ok = dict(x=P(1), w=P(2), K=4, win=P(3), ws=None, qs=1.0, g=P(4), b=P(5), pool=P(6), ss=None,
              n=2, hqk=16, hv=32, dk=128, dv=128, sc=1.0, o=P(7), st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["K"], a["win"], a["ws"], a["qs"], a["g"], a["b"], a["pool"],
                 a["ss"], a["n"], a["hqk"], a["hv"], a["dk"], a["dv"], a["sc"], a["o"], a["st"])

    for name in ("x", "w", "win", "g", "b", "pool", "o"):
        assert call(**{name: None}) == L.GDN_ERR_NULL, name
    assert call(K=1, win=None, n=0) == L.GDN_OK
    assert call(K=0) == L.GDN_ERR_SHAPE
    assert call(K=5) == L.GDN_ERR_UNSUPPORTED
    assert call(hqk=8, hv=32) == L.GDN_ERR_UNSUPPORTED   # four V heads per QK head
    assert call(hv=30) == L.GDN_ERR_SHAPE
    assert call(dk=64) == L.GDN_ERR_UNSUPPORTED
    assert call(n=-1) == L.GDN_ERR_SHAPE
    assert call(n=0) == L.GDN_OK


def test_header_is_plain_c(tmp_path):
    """include/gdn.h compiles as strict C99 (ctypes callers and C code include it)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "use.c"
    src.write_text('#include "gdn.h"\nint main(void) { return (int)GDN_GATE_SILU + (int)GDN_OK; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_binding_fails_loudly_without_library(tmp_path):
    from linear_attention_recurrence_amd import _lib as L
    with pytest.raises(RuntimeError, match="not built"):
        L.load(str(tmp_path / "missing.so"))
