"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module only draws random numbers and stores them in the dtypes and layouts the
library consumes. It holds none of the method's arithmetic, so both the HIP path and the
fp64 oracle can take their inputs from here without sharing any computation.

Distributions (the workload recipe of the Qwen3-Next layer shape; model card "Qwen3-Next",
section "Model Overview": 32 V heads, 16 QK heads, head dim 128):

* q, k ~ N(0, 1), then divided by their L2 norm per token and head; q is *not* scaled here,
  the caller passes ``scale = 128**-0.5`` to the recurrence.
* Large N(0, 1) tensors are drawn by inverse-transform sampling: each value is the standard
  normal quantile at the midpoint of one of 65536 equiprobable cells, picked by a 16-bit
  uniform from PCG64's raw output, and held at bf16 precision. This is a discretised
  N(0, 1) (tails cut at about 4.3 sigma) that is several times faster to draw than
  numpy's ziggurat, which matters for the 2.3-billion-element packed batch.
* v ~ N(0, 1).
* fp32 tensors (q, k, v of an fp32-I/O batch, and every fp32 state) are drawn at full fp32
  precision with numpy's own normal generator, so no fp32 input is exactly representable
  in bf16 by construction (a kernel that rounded one to bf16 would show it).
* beta = sigmoid(N(0, 1)), so beta lies in (0, 1).
* g = log(alpha) = -softplus(N(0, 1)) * 0.1, so alpha lies in (0, 1).
* initial states ~ N(0, 0.02) (0.02 is a standard deviation).
* packed variable-length batches draw lengths uniformly from an inclusive integer range.

bf16 tensors are held as ``numpy.uint16`` bit patterns, rounded from fp32 to nearest even.
Every generator takes a seed and uses numpy's PCG64, so the same call always gives the same
bits.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

D_HEAD = 128
H_QK = 16
H_V = 32
SCALE = D_HEAD ** -0.5


# ----------------------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# ----------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------
# primitive draws
# ----------------------------------------------------------------------------------------

_NORMAL_TABLE = None


def _normal_table() -> np.ndarray:
    """bf16 bits of the N(0,1) quantiles at the midpoints of 65536 equiprobable cells."""
    global _NORMAL_TABLE
    if _NORMAL_TABLE is None:
        from statistics import NormalDist
        inv = NormalDist().inv_cdf
        q = np.array([inv((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float32)
        _NORMAL_TABLE = f32_to_bf16_bits(q)
    return _NORMAL_TABLE


def normal_bf16_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) draws (inverse-transform, 16-bit cells) as bf16 bit patterns."""
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    n = int(np.prod(shape)) if len(shape) else 1
    words = rng.bit_generator.random_raw((n + 3) // 4)
    idx = words.view(np.uint16)[:n]
    return _normal_table()[idx].reshape(shape)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits_to_f32(normal_bf16_bits(rng, shape))


def normal_full_f32(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) draws at full fp32 precision (numpy's normal generator)."""
    return rng.standard_normal(shape, dtype=np.float32)


def _unit_rows(rng: np.random.Generator, shape, full: bool = False) -> np.ndarray:
    """N(0,1) vectors along the last axis, divided by their L2 norm (fp32). `full` draws the
    vectors at full fp32 precision instead of from the bf16-precision table."""
    x = normal_full_f32(rng, shape) if full else normal_f32(rng, shape)
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))[..., None]
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _beta(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _log_alpha(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape).astype(np.float64)
    return (-np.logaddexp(0.0, z) * 0.1).astype(np.float32)


# ----------------------------------------------------------------------------------------
# prefill inputs (packed variable-length sequences)
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillInputs:
    q: np.ndarray               # [T][h_qk][d_k]  uint16 (bf16) or float32
    k: np.ndarray               # [T][h_qk][d_k]
    v: np.ndarray               # [T][h_v][d_v]
    g: np.ndarray               # [T][h_v] float32, log alpha
    beta: np.ndarray            # [T][h_v] float32
    cu_seqlens: np.ndarray      # [N+1] int32
    initial_state: Optional[np.ndarray]  # [N][h_v][d_v][d_k] float32 or None
    scale: float
    io_dtype: str               # "bf16" or "f32"

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def h_qk(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_v(self) -> int:
        return int(self.v.shape[1])

    def as_f64(self, name: str) -> np.ndarray:
        """The exact fp64 value of an input tensor (bf16 bits widened exactly)."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def make_prefill(seq_lens, h_qk=H_QK, h_v=H_V, d_k=D_HEAD, d_v=D_HEAD, io_dtype="bf16",
                 with_initial_state=False, seed=0, scale=None, state_std=0.02) -> PrefillInputs:
    """Packed batch of sequences with the given lengths (zero lengths allowed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = [int(x) for x in seq_lens]
    T = int(sum(seq_lens))
    cu = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seq_lens)
    if io_dtype not in ("bf16", "f32"):
        raise ValueError(io_dtype)
    full = io_dtype == "f32"
    q = _unit_rows(rng, (T, h_qk, d_k), full)
    k = _unit_rows(rng, (T, h_qk, d_k), full)
    v = normal_full_f32(rng, (T, h_v, d_v)) if full else normal_f32(rng, (T, h_v, d_v))
    beta = _beta(rng, (T, h_v))
    g = _log_alpha(rng, (T, h_v))
    s0 = None
    if with_initial_state:
        s0 = normal_full_f32(rng, (len(seq_lens), h_v, d_v, d_k)) * np.float32(state_std)
    if io_dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return PrefillInputs(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, initial_state=s0,
                         scale=float(SCALE if scale is None else scale), io_dtype=io_dtype)


EDGE_CASES = ("no_decay", "strong_decay", "repeated_key", "near_parallel_keys", "zero_rows")


def make_prefill_edge(case: str, seq_lens, h_qk=H_QK, h_v=H_V, io_dtype="bf16",
                      with_initial_state=False, seed=0) -> PrefillInputs:
    """A packed batch drawn as make_prefill, then changed into one of the regimes where the
    update's decay and write strength sit at their limits (page "Qwen3-Next -- How a running
    memory and a searchable history cooperate", section "Correcting a memory instead of
    adding to it": alpha sets how much is kept, beta how hard the key's slot is rewritten):

    * "no_decay": alpha = 1 (g = 0) everywhere;
    * "strong_decay": g = -5 per token, so exp of the running sum underflows fp32 inside a
      64-token block;
    * "repeated_key": beta = 0.999 and, in every 64-token block of each sequence (counted
      from its first token), every token of a QK head carries that block's first key;
    * "near_parallel_keys": beta = 0.999 and keys alternating between two unit vectors whose
      inner product is about 0.999;
    * "zero_rows": tokens 10..20 and 40 of every 64-token block have all-zero k and q rows.

    Only inputs change; nothing of the method is computed here."""
    if case not in EDGE_CASES:
        raise ValueError(case)
    x = make_prefill(seq_lens, h_qk=h_qk, h_v=h_v, io_dtype=io_dtype,
                     with_initial_state=with_initial_state, seed=seed)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    T = x.total_tokens
    cu = x.cu_seqlens
    pos = np.zeros(T, dtype=np.int64)          # position of each token in its sequence
    for n in range(x.num_seqs):
        pos[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])
    as_f32 = (lambda a: bf16_bits_to_f32(a)) if io_dtype == "bf16" else (lambda a: a)
    store = f32_to_bf16_bits if io_dtype == "bf16" else (lambda a: a.astype(np.float32))
    if case == "no_decay":
        x.g = np.zeros_like(x.g)
    elif case == "strong_decay":
        x.g = np.full_like(x.g, -5.0)
    elif case == "repeated_key":
        x.beta = np.full_like(x.beta, 0.999)
        k = as_f32(x.k).copy()
        first = np.arange(T) - (pos % 64)      # token index of each token's block start
        k = k[first]
        x.k = store(k)
    elif case == "near_parallel_keys":
        x.beta = np.full_like(x.beta, 0.999)
        d_k = x.k.shape[2]
        a = _unit_rows(rng, (h_qk, d_k))
        e = _unit_rows(rng, (h_qk, d_k))
        b = a + np.float32(0.045) * (e - np.sum(a * e, axis=-1, keepdims=True) * a)
        b = (b / np.linalg.norm(b, axis=-1, keepdims=True)).astype(np.float32)
        k = np.where((pos % 2 == 0)[:, None, None], a[None], b[None]).astype(np.float32)
        x.k = store(k)
    elif case == "zero_rows":
        z = ((pos % 64 >= 10) & (pos % 64 <= 20)) | (pos % 64 == 40)
        k = as_f32(x.k).copy()
        q = as_f32(x.q).copy()
        k[z] = 0.0
        q[z] = 0.0
        x.k, x.q = store(k), store(q)
    return x


def channel_log_alpha(rows: int, h_v=H_V, d_v=D_HEAD, seed=1007) -> np.ndarray:
    """Per-channel log-decays [rows][h_v][d_v] (float32) for the per-channel form, with the
    distribution of the per-head ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _log_alpha(rng, (rows, h_v, d_v))


def config0(seed=1000) -> PrefillInputs:
    """B=1, T=256, one QK head and one V head, d=128, fp32 everywhere, S0 = 0."""
    return make_prefill([256], h_qk=1, h_v=1, io_dtype="f32", seed=seed)


def config1(seed=1001) -> PrefillInputs:
    """B=1, T=4096, 16 QK / 32 V heads, bf16 q/k/v, S0 = 0 (not passed)."""
    return make_prefill([4096], seed=seed)


def config2(seed=1002) -> PrefillInputs:
    """B=1, T=32768, 16 QK / 32 V heads, bf16 q/k/v, S0 ~ N(0, 0.02)."""
    return make_prefill([32768], with_initial_state=True, seed=seed)


# ----------------------------------------------------------------------------------------
# decode inputs
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    pool: np.ndarray            # [P][h_v][d_v][d_k] float32
    q: np.ndarray               # [R][N][h_qk][d_k] uint16 (ring of R input sets)
    k: np.ndarray               # [R][N][h_qk][d_k]
    v: np.ndarray               # [R][N][h_v][d_v]
    g: np.ndarray               # [R][N][h_v] float32
    beta: np.ndarray            # [R][N][h_v] float32
    slots: Optional[np.ndarray]  # [N] int32 pool slot per sequence, or None (identity)
    scale: float


def make_decode(num_seqs=256, h_qk=H_QK, h_v=H_V, d=D_HEAD, ring=16, pool_size=None,
                permuted_slots=False, seed=1003, state_std=0.02) -> DecodeInputs:
    """A state pool and a ring of per-step single-token inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = num_seqs if pool_size is None else int(pool_size)
    pool = normal_full_f32(rng, (P, h_v, d, d)) * np.float32(state_std)
    q = f32_to_bf16_bits(_unit_rows(rng, (ring, num_seqs, h_qk, d)))
    k = f32_to_bf16_bits(_unit_rows(rng, (ring, num_seqs, h_qk, d)))
    v = normal_bf16_bits(rng, (ring, num_seqs, h_v, d))
    beta = _beta(rng, (ring, num_seqs, h_v))
    g = _log_alpha(rng, (ring, num_seqs, h_v))
    slots = None
    if permuted_slots:
        slots = rng.permutation(P)[:num_seqs].astype(np.int32)
    return DecodeInputs(pool=pool, q=q, k=k, v=v, g=g, beta=beta, slots=slots, scale=SCALE)


def config3(seed=1003) -> DecodeInputs:
    """256 sequences x 1 token, 16 QK / 32 V heads, fp32 pool ~ N(0, 0.02), ring of 16."""
    return make_decode(seed=seed)


# ----------------------------------------------------------------------------------------
# front-end inputs (mixed projected q|k|v channels + conv weights)
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class FrontEndInputs:
    mixed: np.ndarray           # [T][2*h_qk*d_k + h_v*d_v] uint16 (bf16)
    conv_weight: np.ndarray     # [channels][K] float32
    cu_seqlens: np.ndarray      # [N+1] int32
    g: np.ndarray               # [T][h_v] float32
    beta: np.ndarray            # [T][h_v] float32
    initial_state: Optional[np.ndarray]  # [N][h_v][d_v][d_k] float32
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    q_scale: float

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1)


def make_frontend(seq_lens, h_qk=H_QK, h_v=H_V, d_k=D_HEAD, d_v=D_HEAD, conv_kernel=4,
                  with_initial_state=True, seed=1004, block_rows=1 << 16) -> FrontEndInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = [int(x) for x in seq_lens]
    T = int(sum(seq_lens))
    cu = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seq_lens)
    C = 2 * h_qk * d_k + h_v * d_v
    mixed = np.empty((T, C), dtype=np.uint16)
    for r0 in range(0, T, block_rows):   # bounded temporaries for large batches
        r1 = min(T, r0 + block_rows)
        mixed[r0:r1] = normal_bf16_bits(rng, (r1 - r0, C))
    w = (rng.standard_normal((C, conv_kernel), dtype=np.float32) * np.float32(0.1))
    beta = _beta(rng, (T, h_v))
    g = _log_alpha(rng, (T, h_v))
    s0 = None
    if with_initial_state:
        s0 = normal_full_f32(rng, (len(seq_lens), h_v, d_v, d_k)) * np.float32(0.02)
    return FrontEndInputs(mixed=mixed, conv_weight=w, cu_seqlens=cu, g=g, beta=beta,
                          initial_state=s0, h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v,
                          q_scale=float(d_k ** -0.5))


def config4_lengths(seed=1004, num_seqs=64, lo=128, hi=8192):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(lo, hi, size=num_seqs, endpoint=True)]


def config4(seed=1004) -> FrontEndInputs:
    """64 sequences, lengths uniform in [128, 8192], mixed bf16 [sum T][8192], conv k=4."""
    return make_frontend(config4_lengths(seed), seed=seed + 100)


def epilogue_inputs(rows: int, h_v: int = H_V, d_v: int = D_HEAD, io_dtype: str = "bf16",
                    seed: int = 1012):
    """Inputs of the output epilogue: a read-out o whose (token, head) vectors span eight
    e-folds of size (as a mixer's read-out does across heads and positions), a gate input z
    ~ N(0, 3^2) and a small zero-centred scale w ~ N(0, 0.1^2) [d_v] fp32. o and z are bf16
    bit patterns for io_dtype "bf16", else fp32. Returns (o, z, w)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    o = rng.standard_normal((rows, h_v, d_v)) * np.exp(rng.uniform(-6, 2, (rows, h_v, 1)))
    z = rng.standard_normal((rows, h_v, d_v)) * 3.0
    w = (rng.standard_normal(d_v) * 0.1).astype(np.float32)
    if io_dtype == "bf16":
        return f32_to_bf16_bits(o.astype(np.float32)), f32_to_bf16_bits(z.astype(np.float32)), w
    return o.astype(np.float32), z.astype(np.float32), w
