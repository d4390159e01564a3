"""ctypes binding of libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream; every step of the computation runs in the library's HIP kernels. There is no CPU
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the library to load (for instance one with the host
# code built under the address and undefined-behaviour sanitizers).
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(6)
GDN_BF16, GDN_F32 = 0, 1

EXPORTED = ("gdn_status_string", "gdn_chunk_prefill_workspace_bytes", "gdn_chunk_prefill",
            "gdn_decode_step", "gdn_verify_step", "gdn_channel_decay_prefill",
            "gdn_channel_decay_decode_step", "gdn_conv_prep", "gdn_conv_decode_step",
            "gdn_conv_window_from_prefill", "gdn_gated_rmsnorm", "gdn_decode_step_with_conv",
            "gdn_chunk_prefill_noalloc", "gdn_chunk_prefill_conv_workspace_bytes",
            "gdn_chunk_prefill_conv")

NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, gdn_status_string(status)))


def load(path: Optional[str] = None):
    """Load libgdn.so and declare the signatures. Raises if the library is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libgdn.so is not built at %s; run "
                           "linear_attention_recurrence_amd.build.build()" % p)
    lib = ctypes.CDLL(p)
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_chunk_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_prefill_workspace_bytes.argtypes = [_I] * 6
    lib.gdn_chunk_prefill.restype = ctypes.c_int
    lib.gdn_chunk_prefill.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _I, _I, _I, _I, _I,
                                      _I, ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_chunk_prefill_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_prefill_conv_workspace_bytes.argtypes = [_I] * 6
    lib.gdn_chunk_prefill_conv.restype = ctypes.c_int
    lib.gdn_chunk_prefill_conv.argtypes = [_P, _P, _I, ctypes.c_float, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                           ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_chunk_prefill_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_prefill_noalloc.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _I, _I, _I, _I,
                                              _I, _I, ctypes.c_float, _P, _P, _P, _P]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _P, _I, _I, _I, _I,
                                    _I, ctypes.c_float, _P, _P]
    lib.gdn_verify_step.restype = ctypes.c_int
    lib.gdn_verify_step.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                    _I, _I, ctypes.c_float, _P, _P]
    lib.gdn_channel_decay_prefill.restype = ctypes.c_int
    lib.gdn_channel_decay_prefill.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _I, _I, _I, _I,
                                              _I, _I, ctypes.c_float, _P, _P, _P, _P]
    lib.gdn_channel_decay_decode_step.restype = ctypes.c_int
    lib.gdn_channel_decay_decode_step.argtypes = lib.gdn_decode_step.argtypes
    lib.gdn_conv_prep.restype = ctypes.c_int
    lib.gdn_conv_prep.argtypes = [_P, _P, _I, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                                  _P, _P, _P, _P]
    lib.gdn_conv_decode_step.restype = ctypes.c_int
    lib.gdn_conv_decode_step.argtypes = [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float,
                                         _P, _P, _P, _P]
    lib.gdn_conv_window_from_prefill.restype = ctypes.c_int
    lib.gdn_conv_window_from_prefill.argtypes = [_P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]
    lib.gdn_decode_step_with_conv.restype = ctypes.c_int
    lib.gdn_decode_step_with_conv.argtypes = [_P, _P, _I, _P, _P, ctypes.c_float, _P, _P, _P, _P,
                                              _I, _I, _I, _I, _I, ctypes.c_float, _P, _P]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [_P, _P, ctypes.c_int, _P, _I, _I, _I, ctypes.c_float,
                                      ctypes.c_int, _P, _P]
    if path is None:
        _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgdn must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _on(stream):
    """Allocation context for a call launched on `stream`: tensors the binding allocates
    (outputs, the prefill workspace) then belong to that stream in torch's caching
    allocator, so their memory is not handed to work queued on another stream while the
    call's kernels may still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise ValueError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _expect(t, shape, dtype, name):
    """Shape/dtype/device check of one argument (so a kernel never indexes past a buffer)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)


def _check(status: int, where: str):
    if status != GDN_OK:
        raise GdnError(status, where)


def gdn_chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v) -> int:
    return int(load().gdn_chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v))


def gdn_chunk_prefill(q, k, v, g, beta, cu_seqlens, scale, initial_state=None,
                      final_state=None, o=None, workspace=None, stream=None):
    """o = prefill over a packed batch. Shapes: q, k [T][h_qk][d_k]; v [T][h_v][d_v];
    g, beta [T][h_v] fp32; cu_seqlens [N+1] int32; states [N][h_v][d_v][d_k] fp32.
    Returns o (allocated with torch.empty when not given)."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    with _on(stream):
        if o is None:
            o = torch.empty((T, h_v, d_v), dtype=v.dtype, device=v.device)
        need = gdn_chunk_prefill_workspace_bytes(T, N, h_qk, h_v, d_k, d_v)
        if need and workspace is None and q.dtype == torch.bfloat16:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _expect(k, (T, h_qk, d_k), q.dtype, "k")
    _expect(v, (T, h_v, d_v), q.dtype, "v")
    _expect(g, (T, h_v), torch.float32, "g")
    _expect(beta, (T, h_v), torch.float32, "beta")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _expect(initial_state, (N, h_v, d_v, d_k), torch.float32, "initial_state")
    _expect(final_state, (N, h_v, d_v, d_k), torch.float32, "final_state")
    _expect(o, (T, h_v, d_v), q.dtype, "o")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gdn_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                                  _ptr(cu_seqlens), N, T, h_qk, h_v, d_k, d_v, float(scale),
                                  _ptr(initial_state), _ptr(final_state), _ptr(o),
                                  _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_prefill")
    return o


def gdn_chunk_prefill_conv_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v) -> int:
    return int(load().gdn_chunk_prefill_conv_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v))


def gdn_chunk_prefill_conv(mixed_qkv, conv_weight, g, beta, cu_seqlens, h_qk, h_v, d_k, d_v, q_scale,
                           scale, initial_state=None, final_state=None, o=None, workspace=None,
                           stream=None):
    """The front end (gdn_conv_prep) and the prefill in one call, from the mixed bf16 input
    [T][2 h_qk d_k + h_v d_v] and the conv taps [channels][K] fp32. Returns o [T][h_v][d_v] bf16."""
    T, C = mixed_qkv.shape
    N = cu_seqlens.numel() - 1
    K = int(conv_weight.shape[1])
    with _on(stream):
        if o is None:
            o = torch.empty((T, h_v, d_v), dtype=torch.bfloat16, device=mixed_qkv.device)
        need = gdn_chunk_prefill_conv_workspace_bytes(T, N, h_qk, h_v, d_k, d_v)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=mixed_qkv.device)
    _expect(mixed_qkv, (T, 2 * h_qk * d_k + h_v * d_v), torch.bfloat16, "mixed_qkv")
    _expect(conv_weight, (C, K), torch.float32, "conv_weight")
    _expect(g, (T, h_v), torch.float32, "g")
    _expect(beta, (T, h_v), torch.float32, "beta")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _expect(initial_state, (N, h_v, d_v, d_k), torch.float32, "initial_state")
    _expect(final_state, (N, h_v, d_v, d_k), torch.float32, "final_state")
    _expect(o, (T, h_v, d_v), torch.bfloat16, "o")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gdn_chunk_prefill_conv(_ptr(mixed_qkv), _ptr(conv_weight), K, float(q_scale), _ptr(g),
                                       _ptr(beta), _ptr(cu_seqlens), N, T, h_qk, h_v, d_k, d_v,
                                       float(scale), _ptr(initial_state), _ptr(final_state), _ptr(o),
                                       _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_prefill_conv")
    return o


def gdn_chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, scale, o, initial_state=None,
                              final_state=None, stream=None):
    """gdn_chunk_prefill with its workspace in the library's own device scratch: nothing is
    allocated, here or in the library, so o must be given. Shapes as gdn_chunk_prefill.
    Returns o."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    _expect(k, (T, h_qk, d_k), q.dtype, "k")
    _expect(v, (T, h_v, d_v), q.dtype, "v")
    _expect(g, (T, h_v), torch.float32, "g")
    _expect(beta, (T, h_v), torch.float32, "beta")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _expect(initial_state, (N, h_v, d_v, d_k), torch.float32, "initial_state")
    _expect(final_state, (N, h_v, d_v, d_k), torch.float32, "final_state")
    _expect(o, (T, h_v, d_v), q.dtype, "o")
    st = load().gdn_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                          _ptr(beta), _ptr(cu_seqlens), N, T, h_qk, h_v, d_k, d_v,
                                          float(scale), _ptr(initial_state), _ptr(final_state),
                                          _ptr(o), _stream(stream))
    _check(st, "gdn_chunk_prefill_noalloc")
    return o


def gdn_decode_step(q, k, v, g, beta, state_pool, scale, state_slots=None, o=None, stream=None):
    """One token per sequence; state_pool [P][h_v][d_v][d_k] fp32 is updated in place.
    Returns o [N][h_v][d_v]."""
    N, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if o is None:
        with _on(stream):
            o = torch.empty((N, h_v, d_v), dtype=v.dtype, device=v.device)
    _expect(k, (N, h_qk, d_k), q.dtype, "k")
    _expect(v, (N, h_v, d_v), q.dtype, "v")
    _expect(g, (N, h_v), torch.float32, "g")
    _expect(beta, (N, h_v), torch.float32, "beta")
    _expect(state_pool, (state_pool.shape[0], h_v, d_v, d_k), torch.float32, "state_pool")
    _expect(o, (N, h_v, d_v), q.dtype, "o")
    if state_slots is None:
        if state_pool.shape[0] < N:
            raise ValueError("state_pool has fewer entries than sequences")
    else:
        _expect(state_slots, (N,), torch.int32, "state_slots")
    st = load().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                                _ptr(state_pool), _ptr(state_slots), N, h_qk, h_v, d_k, d_v,
                                float(scale), _ptr(o), _stream(stream))
    _check(st, "gdn_decode_step")
    return o


def gdn_verify_step(q, k, v, g, beta, state_pool, scale, state_slots=None, snapshots=None,
                    o=None, stream=None):
    """num_tokens decode steps per sequence in one call (q [N][n_tok][h_qk][d_k], ...);
    state_pool is updated in place to the state after the last token, and snapshots
    [N][n_tok][h_v][d_v][d_k] fp32, if given, receives the state after each token. Returns
    o [N][n_tok][h_v][d_v]."""
    N, n_tok, h_qk, d_k = q.shape
    h_v, d_v = v.shape[2], v.shape[3]
    if o is None:
        with _on(stream):
            o = torch.empty((N, n_tok, h_v, d_v), dtype=v.dtype, device=v.device)
    _expect(k, (N, n_tok, h_qk, d_k), q.dtype, "k")
    _expect(v, (N, n_tok, h_v, d_v), q.dtype, "v")
    _expect(g, (N, n_tok, h_v), torch.float32, "g")
    _expect(beta, (N, n_tok, h_v), torch.float32, "beta")
    _expect(state_pool, (state_pool.shape[0], h_v, d_v, d_k), torch.float32, "state_pool")
    _expect(o, (N, n_tok, h_v, d_v), q.dtype, "o")
    if snapshots is not None:
        _expect(snapshots, (N, n_tok, h_v, d_v, d_k), torch.float32, "snapshots")
    if state_slots is None:
        if state_pool.shape[0] < N:
            raise ValueError("state_pool has fewer entries than sequences")
    else:
        _expect(state_slots, (N,), torch.int32, "state_slots")
    st = load().gdn_verify_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                                _ptr(state_pool), _ptr(state_slots), _ptr(snapshots), N, n_tok,
                                h_qk, h_v, d_k, d_v, float(scale), _ptr(o), _stream(stream))
    _check(st, "gdn_verify_step")
    return o


def gdn_channel_decay_prefill(q, k, v, g, beta, cu_seqlens, scale, initial_state=None,
                              final_state=None, o=None, stream=None):
    """The per-channel form over a packed batch; g [T][h_v][d_v]. Returns o."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if o is None:
        with _on(stream):
            o = torch.empty((T, h_v, d_v), dtype=v.dtype, device=v.device)
    _expect(k, (T, h_qk, d_k), q.dtype, "k")
    _expect(v, (T, h_v, d_v), q.dtype, "v")
    _expect(g, (T, h_v, d_v), torch.float32, "g")
    _expect(beta, (T, h_v), torch.float32, "beta")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _expect(o, (T, h_v, d_v), q.dtype, "o")
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        if st is not None:
            _expect(st, (N, h_v, d_v, d_k), torch.float32, name)
    st = load().gdn_channel_decay_prefill(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                          _ptr(beta), _ptr(cu_seqlens), N, T, h_qk, h_v, d_k, d_v,
                                          float(scale), _ptr(initial_state), _ptr(final_state),
                                          _ptr(o), _stream(stream))
    _check(st, "gdn_channel_decay_prefill")
    return o


def gdn_channel_decay_decode_step(q, k, v, g, beta, state_pool, scale, state_slots=None, o=None,
                                  stream=None):
    """The per-channel form at one token per sequence; g [N][h_v][d_v]; state_pool is
    updated in place. Returns o."""
    N, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if o is None:
        with _on(stream):
            o = torch.empty((N, h_v, d_v), dtype=v.dtype, device=v.device)
    _expect(k, (N, h_qk, d_k), q.dtype, "k")
    _expect(v, (N, h_v, d_v), q.dtype, "v")
    _expect(g, (N, h_v, d_v), torch.float32, "g")
    _expect(beta, (N, h_v), torch.float32, "beta")
    _expect(state_pool, (state_pool.shape[0], h_v, d_v, d_k), torch.float32, "state_pool")
    _expect(o, (N, h_v, d_v), q.dtype, "o")
    if state_slots is None:
        if state_pool.shape[0] < N:
            raise ValueError("state_pool has fewer entries than sequences")
    else:
        _expect(state_slots, (N,), torch.int32, "state_slots")
    st = load().gdn_channel_decay_decode_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                              _ptr(beta), _ptr(state_pool), _ptr(state_slots), N,
                                              h_qk, h_v, d_k, d_v, float(scale), _ptr(o),
                                              _stream(stream))
    _check(st, "gdn_channel_decay_decode_step")
    return o


def gdn_conv_prep(mixed_qkv, conv_weight, cu_seqlens, h_qk, h_v, d_k, d_v, q_scale,
                  q=None, k=None, v=None, stream=None):
    """Front end; returns (q, k, v) bf16 tensors laid out as the prefill inputs."""
    T = mixed_qkv.shape[0]
    N = cu_seqlens.numel() - 1
    dev = mixed_qkv.device
    with _on(stream):
        if q is None:
            q = torch.empty((T, h_qk, d_k), dtype=torch.bfloat16, device=dev)
        if k is None:
            k = torch.empty((T, h_qk, d_k), dtype=torch.bfloat16, device=dev)
        if v is None:
            v = torch.empty((T, h_v, d_v), dtype=torch.bfloat16, device=dev)
    C = 2 * h_qk * d_k + h_v * d_v
    _expect(mixed_qkv, (T, C), torch.bfloat16, "mixed_qkv")
    _expect(conv_weight, (C, conv_weight.shape[1]), torch.float32, "conv_weight")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _expect(q, (T, h_qk, d_k), torch.bfloat16, "q")
    _expect(k, (T, h_qk, d_k), torch.bfloat16, "k")
    _expect(v, (T, h_v, d_v), torch.bfloat16, "v")
    st = load().gdn_conv_prep(_ptr(mixed_qkv), _ptr(conv_weight), int(conv_weight.shape[1]),
                              _ptr(cu_seqlens), N, T, h_qk, h_v, d_k, d_v, float(q_scale),
                              _ptr(q), _ptr(k), _ptr(v), _stream(stream))
    _check(st, "gdn_conv_prep")
    return q, k, v


def gdn_conv_decode_step(mixed_qkv, conv_weight, conv_window, h_qk, h_v, d_k, d_v, q_scale,
                         window_slots=None, q=None, k=None, v=None, stream=None):
    """Front end for one token per sequence; conv_window [P][K-1][C] bf16 is updated in
    place. Returns (q, k, v) laid out as the decode-step inputs."""
    N = mixed_qkv.shape[0]
    K = int(conv_weight.shape[1])
    dev = mixed_qkv.device
    with _on(stream):
        if q is None:
            q = torch.empty((N, h_qk, d_k), dtype=torch.bfloat16, device=dev)
        if k is None:
            k = torch.empty((N, h_qk, d_k), dtype=torch.bfloat16, device=dev)
        if v is None:
            v = torch.empty((N, h_v, d_v), dtype=torch.bfloat16, device=dev)
    C = 2 * h_qk * d_k + h_v * d_v
    _expect(mixed_qkv, (N, C), torch.bfloat16, "mixed_qkv")
    _expect(conv_weight, (C, K), torch.float32, "conv_weight")
    if K > 1:
        _expect(conv_window, (conv_window.shape[0], K - 1, C), torch.bfloat16, "conv_window")
        if window_slots is None and conv_window.shape[0] < N:
            raise ValueError("conv_window has fewer slots than sequences")
    if window_slots is not None:
        _expect(window_slots, (N,), torch.int32, "window_slots")
    _expect(q, (N, h_qk, d_k), torch.bfloat16, "q")
    _expect(k, (N, h_qk, d_k), torch.bfloat16, "k")
    _expect(v, (N, h_v, d_v), torch.bfloat16, "v")
    st = load().gdn_conv_decode_step(_ptr(mixed_qkv), _ptr(conv_weight), K,
                                     _ptr(conv_window) if K > 1 else None, _ptr(window_slots), N,
                                     h_qk, h_v, d_k, d_v, float(q_scale), _ptr(q), _ptr(k), _ptr(v),
                                     _stream(stream))
    _check(st, "gdn_conv_decode_step")
    return q, k, v


def gdn_conv_window_from_prefill(mixed_qkv, conv_kernel, cu_seqlens, conv_window, h_qk, h_v,
                                 d_k, d_v, window_slots=None, stream=None):
    """Writes each sequence's last conv_kernel-1 inputs (zeros before its start) into its
    slot of conv_window [P][conv_kernel-1][C] bf16."""
    T = mixed_qkv.shape[0]
    N = cu_seqlens.numel() - 1
    K = int(conv_kernel)
    C = 2 * h_qk * d_k + h_v * d_v
    _expect(mixed_qkv, (T, C), torch.bfloat16, "mixed_qkv")
    _expect(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    if K > 1:
        _expect(conv_window, (conv_window.shape[0], K - 1, C), torch.bfloat16, "conv_window")
        if window_slots is None and conv_window.shape[0] < N:
            raise ValueError("conv_window has fewer slots than sequences")
    if window_slots is not None:
        _expect(window_slots, (N,), torch.int32, "window_slots")
    st = load().gdn_conv_window_from_prefill(_ptr(mixed_qkv), K, _ptr(cu_seqlens), N, T, h_qk, h_v,
                                             d_k, d_v, _ptr(conv_window) if K > 1 else None,
                                             _ptr(window_slots), _stream(stream))
    _check(st, "gdn_conv_window_from_prefill")


GATES = {"sigmoid": 0, "silu": 1}


def gdn_gated_rmsnorm(o, z, weight, eps=1e-6, gate="sigmoid", out=None, stream=None):
    """Output epilogue: per V head, o / rms(o) * (1 + weight) * gate(z). o, z [T][h_v][d_v]
    (bf16 or fp32, same dtype); weight [d_v] fp32; gate "sigmoid" or "silu". out may be o
    or z (in place). Returns out."""
    T, h_v, d_v = o.shape
    if out is None:
        with _on(stream):
            out = torch.empty_like(o)
    _expect(z, (T, h_v, d_v), o.dtype, "z")
    _expect(weight, (d_v,), torch.float32, "weight")
    _expect(out, (T, h_v, d_v), o.dtype, "out")
    if gate not in GATES:
        raise ValueError("gate must be one of %s" % sorted(GATES))
    st = load().gdn_gated_rmsnorm(_ptr(o), _ptr(z), _dtype_code(o), _ptr(weight), T, h_v, d_v,
                                  float(eps), GATES[gate], _ptr(out), _stream(stream))
    _check(st, "gdn_gated_rmsnorm")
    return out


def gdn_decode_step_with_conv(mixed_qkv, conv_weight, conv_window, g, beta, state_pool, h_qk, h_v,
                              d_k, d_v, q_scale, scale, window_slots=None, state_slots=None,
                              o=None, stream=None):
    """gdn_conv_decode_step then gdn_decode_step in one launch (bit for bit the same results);
    mixed_qkv [N][C] bf16, conv_weight [C][K] fp32, conv_window [P][K-1][C] bf16 (or None for
    K = 1), g, beta [N][h_v] fp32, state_pool [P'][h_v][d_v][d_k] fp32. Returns o
    [N][h_v][d_v] bf16."""
    N, C = mixed_qkv.shape
    K = conv_weight.shape[1]
    if o is None:
        with _on(stream):
            o = torch.empty((N, h_v, d_v), dtype=torch.bfloat16, device=mixed_qkv.device)
    _expect(mixed_qkv, (N, 2 * h_qk * d_k + h_v * d_v), torch.bfloat16, "mixed_qkv")
    _expect(conv_weight, (C, K), torch.float32, "conv_weight")
    if conv_window is not None:
        _expect(conv_window, (conv_window.shape[0], K - 1, C), torch.bfloat16, "conv_window")
    _expect(g, (N, h_v), torch.float32, "g")
    _expect(beta, (N, h_v), torch.float32, "beta")
    _expect(state_pool, (state_pool.shape[0], h_v, d_v, d_k), torch.float32, "state_pool")
    _expect(o, (N, h_v, d_v), torch.bfloat16, "o")
    for name, sl in (("window_slots", window_slots), ("state_slots", state_slots)):
        if sl is not None:
            _expect(sl, (N,), torch.int32, name)
    st = load().gdn_decode_step_with_conv(_ptr(mixed_qkv), _ptr(conv_weight), K, _ptr(conv_window),
                                          _ptr(window_slots), float(q_scale), _ptr(g), _ptr(beta),
                                          _ptr(state_pool), _ptr(state_slots), N, h_qk, h_v, d_k,
                                          d_v, float(scale), _ptr(o), _stream(stream))
    _check(st, "gdn_decode_step_with_conv")
    return o
