/*
 * gdn.h -- C ABI of libgdn.so, a Gated DeltaNet token mixer for AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Qwen3-Next -- How a running memory and a searchable history
 * cooperate", section "Correcting a memory instead of adding to it"): each V head keeps a
 * fixed d_v x d_k state S. For every token it first shrinks S by a decay alpha, then
 * corrects what S returns for the key k toward the value v with write strength beta:
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 * and the layer output is o_t = scale * S_t q_t, read after the update (token loop in
 * section "01 . GatedDeltaNet(config)" of page "Qwen3-Next 80B-A3B -- The Evolving
 * Transformer"). alpha is passed as its logarithm g = log(alpha). The state size does not
 * depend on the number of tokens (section "Two kinds of remembering" of the first page).
 *
 * Heads (model card "Qwen3-Next", section "Model Overview"): h_qk query/key heads are shared
 * by h_v value heads; V head h reads QK head h / (h_v / h_qk). The library supports
 * d_k = d_v = 128 (the model's head dim) and any h_qk, h_v with h_v % h_qk == 0.
 *
 * Conventions for every function:
 *  - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent). Layouts are row-major
 *    and contiguous, last index fastest. bf16 is the IEEE-style 16-bit brain float.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the default
 *    stream). The library never allocates, frees or synchronises, and keeps no global
 *    mutable state: calls are re-entrant and thread-safe.
 *  - The caller owns every buffer. Arguments are validated on the host before anything is
 *    launched; on a nonzero status nothing has been written. A failed launch returns
 *    GDN_ERR_HIP. Nothing is thrown across the ABI.
 *  - Device-side contracts that the host cannot check without a synchronisation:
 *    cu_seqlens is nondecreasing from 0 to total_tokens; state_slots (and window_slots)
 *    hold distinct indices below the pool size; every log-decay g is finite and <= 0, i.e.
 *    alpha = exp(g) lies in (0, 1] (a decay shrinks the state, as the first page's section
 *    "Correcting a memory instead of adding to it" describes it). Breaking them is
 *    undefined behaviour: for g > 0 the chunked prefill bounds every in-chunk decay ratio
 *    by 1 while the token-sequential kernels do not, so the two would disagree. For
 *    debugging a caller, the environment variable GDN_CHECK_CONTRACTS=1 makes every call
 *    copy these arrays to the host on its stream and wait for them (the one case where the
 *    library synchronises), and return GDN_ERR_SHAPE, with nothing launched, for a
 *    cu_seqlens that does not start at 0, decreases or does not end at total_tokens, for
 *    negative or repeated slots (the pool size is not passed, so its bound stays the
 *    caller's), or for a g that is positive, infinite or NaN. A failed copy returns
 *    GDN_ERR_HIP.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,        /* a size is negative or inconsistent */
    GDN_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head dim != 128, dtype, ...) */
    GDN_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the query says */
    GDN_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} gdn_status;

typedef enum {
    GDN_BF16 = 0,             /* q, k, v and o in bf16; arithmetic in fp32 */
    GDN_F32 = 1               /* q, k, v and o in fp32; arithmetic in fp32 */
} gdn_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* gdn_status_string(gdn_status s);

/*
 * Bytes of device workspace gdn_chunk_prefill needs (io_dtype GDN_BF16) for these sizes: for
 * every 64-token chunk, 25600 bytes per V head (decay factors, and T diag(beta) =
 * (I + A)^-1 diag(beta) and the masked and decayed Q K^T each as a hi + lo bf16 pair),
 * sized for ceil(total_tokens / 64) + num_seqs chunks so no host read of cu_seqlens is
 * needed. With at most 64 (sequence, V head) pairs the call instead runs in segments of 64
 * chunks per sequence whenever that needs less: num_seqs * (64 * h_v * 25600 + h_v * d_v *
 * d_k * 4) bytes (one segment's blocks and the states between segments), whatever the
 * lengths -- 54.5 MB for one sequence at 32 V heads, 109 MB for two. With total_tokens = 0
 * (every sequence empty) no workspace is needed: 0, and workspace may be NULL.
 * Returns 0 for invalid sizes. The contents are scratch: nothing persists between calls,
 * and calls sharing a workspace must not overlap.
 */
size_t gdn_chunk_prefill_workspace_bytes(int32_t total_tokens, int32_t num_seqs,
                                         int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v);

/*
 * Prefill: runs the gated delta rule over a packed batch of variable-length sequences.
 *
 *   q, k          [total_tokens][h_qk][d_k]      io_dtype
 *   v             [total_tokens][h_v][d_v]       io_dtype
 *   g, beta       [total_tokens][h_v]            fp32; alpha = exp(g), g finite and <= 0
 *   cu_seqlens    [num_seqs + 1]                 int32; sequence n spans tokens
 *                                                cu_seqlens[n] .. cu_seqlens[n+1]-1
 *   scale         multiplies the read-out (o = scale * S q)
 *   initial_state [num_seqs][h_v][d_v][d_k] fp32, or NULL for zero states
 *   final_state   same shape, or NULL to skip; may alias initial_state (in-place update)
 *   o             [total_tokens][h_v][d_v]       io_dtype
 *   workspace     at least gdn_chunk_prefill_workspace_bytes(...) bytes (unused, may be
 *                 NULL, for GDN_F32)
 *
 * Zero-length sequences are allowed: their final state is their initial state.
 * io_dtype GDN_BF16 runs the chunked kernel (chunks of 64 tokens; intra-chunk products on
 * bf16 matrix cores with fp32 accumulation, the state carried in fp32). GDN_F32 runs a
 * token-sequential fp32 kernel (for fp32 inputs whose products must not round to bf16).
 */
gdn_status gdn_chunk_prefill(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                             const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                             int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                             const float* initial_state, float* final_state,
                             void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill from the layer's projected input: the front end of gdn_conv_prep (the short causal
 * depthwise convolution that section "01 . GatedDeltaNet(config)" of page "Qwen3-Next 80B-A3B
 * -- The Evolving Transformer" places before the recurrence, SiLU, the L2 norm of each q and
 * k head and q_scale) followed by gdn_chunk_prefill, in one call, bit for bit equal to those
 * two calls.
 *
 *   mixed_qkv     [total_tokens][2 h_qk d_k + h_v d_v] bf16, channels q | k | v, head-major
 *   conv_weight   [channels][conv_kernel] fp32, tap conv_kernel - 1 on the current token;
 *                 1 <= conv_kernel <= 4
 *   q_scale       multiplies the normalised q (the front end's scale); `scale` multiplies
 *                 the read-out as in gdn_chunk_prefill (1 when q_scale already holds d_k^-1/2)
 *   g, beta, cu_seqlens, states, o (bf16) as gdn_chunk_prefill
 *   workspace     at least gdn_chunk_prefill_conv_workspace_bytes(...) bytes
 *
 * The front end runs as its own pass into the workspace (q, k and v after the prefill's own
 * blocks, which the size query includes), then the prefill reads them there: the results are
 * bit for bit those of gdn_conv_prep followed by gdn_chunk_prefill.
 * Validation and errors as gdn_chunk_prefill and gdn_conv_prep.
 */
size_t gdn_chunk_prefill_conv_workspace_bytes(int32_t total_tokens, int32_t num_seqs,
                                              int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v);
gdn_status gdn_chunk_prefill_conv(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                                  float q_scale, const float* g, const float* beta,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                  int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                                  const float* initial_state, float* final_state, void* o,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's own device scratch behind gdn_chunk_prefill_noalloc (per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gdn_chunk_prefill for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same operation,
 * arguments and results as gdn_chunk_prefill (bit for bit: the same kernels), without the
 * workspace arguments: the workspace is a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held from the first such call on that GPU until the
 * process ends. The call allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine); the caller still owns q, k, v, g, beta, cu_seqlens, the states and o.
 *
 * Limit: sizes for which gdn_chunk_prefill_workspace_bytes(...) exceeds
 * GDN_NOALLOC_SCRATCH_BYTES return GDN_ERR_WORKSPACE with nothing launched. One sequence at
 * 32 V heads (or any batch of up to 64 (sequence, V head) pairs needing at most the
 * scratch in segments, i.e. up to 39 pairs) has no length limit; larger batches at 32 V
 * heads need ceil(total_tokens / 64) + num_seqs <= 81, e.g. two sequences of 2,528 tokens
 * each.
 * GDN_F32 needs no workspace and has no limit.
 *
 * Sharing: every call on one GPU uses that GPU's one array, which keeps whatever the last
 * call left in it; nothing in it needs to start at zero (each call writes every byte of it
 * that it later reads). Calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race on the array and give undefined results; calls
 * ordered on one stream, or on different GPUs, are safe. The first call on a GPU looks up
 * that GPU's copy of the array (hipGetSymbolAddress); a failure there returns GDN_ERR_HIP.
 */
gdn_status gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t total_tokens, int32_t h_qk, int32_t h_v, int32_t d_k,
                                     int32_t d_v, float scale, const float* initial_state,
                                     float* final_state, void* o, void* stream);

/*
 * Decode: one token for each of num_seqs sequences, updating their states in place.
 *
 *   q, k          [num_seqs][h_qk][d_k]          io_dtype
 *   v             [num_seqs][h_v][d_v]           io_dtype
 *   g, beta       [num_seqs][h_v]                fp32
 *   state_pool    [pool_size][h_v][d_v][d_k]     fp32, read and written in place
 *   state_slots   [num_seqs] int32: sequence n uses pool entry state_slots[n]; NULL means
 *                 entry n. Slots must be distinct.
 *   o             [num_seqs][h_v][d_v]           io_dtype
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                           const float* g, const float* beta,
                           float* state_pool, const int32_t* state_slots,
                           int32_t num_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                           float scale, void* o, void* stream);

/*
 * Verify: num_tokens decode steps for each of num_seqs sequences in one call -- the draft
 * tokens of a speculative step, which the main model checks together and keeps as far as it
 * agrees (page "Qwen3-Next -- How a running memory and a searchable history cooperate",
 * section "Speed depends on the serving software"). Token t of sequence n is the t-th step of
 * gdn_decode_step for that sequence, with the same arithmetic, so the outputs and states are
 * bit for bit those of num_tokens successive gdn_decode_step calls. The state is read once
 * and written once; with snapshots set, the state after every token is kept as well, so a
 * caller that accepts only the first m drafts can restore snapshot m-1.
 *
 *   q, k          [num_seqs][num_tokens][h_qk][d_k]   io_dtype
 *   v             [num_seqs][num_tokens][h_v][d_v]    io_dtype
 *   g, beta       [num_seqs][num_tokens][h_v]         fp32
 *   state_pool    [pool_size][h_v][d_v][d_k] fp32, read and written in place: on return it
 *                 holds each sequence's state after its last token
 *   state_slots   [num_seqs] int32, as for gdn_decode_step (NULL: entry n); distinct
 *   snapshots     [num_seqs][num_tokens][h_v][d_v][d_k] fp32: the state after each token,
 *                 or NULL to keep none
 *   o             [num_seqs][num_tokens][h_v][d_v]    io_dtype
 */
gdn_status gdn_verify_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                           const float* g, const float* beta,
                           float* state_pool, const int32_t* state_slots, float* snapshots,
                           int32_t num_seqs, int32_t num_tokens, int32_t h_qk, int32_t h_v,
                           int32_t d_k, int32_t d_v, float scale, void* o, void* stream);

/*
 * The per-channel form of the rule, as the code panel of section "01 . GatedDeltaNet(config)"
 * of page "Qwen3-Next 80B-A3B -- The Evolving Transformer" writes it: one decay per value
 * channel (row i of S), and the correction measured against the state before the decay:
 *
 *     S_t = diag(alpha_t) S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,   o_t = scale * S_t q_t
 *
 * Each value row then has its own transition, so these run token by token (no chunked
 * form); arithmetic in fp32, states in fp32.
 *
 * Prefill over a packed batch, arguments as for gdn_chunk_prefill except
 *   g             [total_tokens][h_v][d_v] fp32: log alpha per token, V head and value channel
 * and no workspace (none is used).
 */
gdn_status gdn_channel_decay_prefill(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                     int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                                     const float* initial_state, float* final_state, void* o,
                                     void* stream);

/*
 * The per-channel form at one token per sequence over a state pool, in place; arguments as
 * for gdn_decode_step except
 *   g             [num_seqs][h_v][d_v] fp32: log alpha per V head and value channel
 */
gdn_status gdn_channel_decay_decode_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                         const float* g, const float* beta,
                                         float* state_pool, const int32_t* state_slots,
                                         int32_t num_seqs, int32_t h_qk, int32_t h_v, int32_t d_k,
                                         int32_t d_v, float scale, void* o, void* stream);

/*
 * Front end: short causal depthwise convolution, SiLU, L2 normalisation of every q and k
 * head, and a scale on q (section "01 . GatedDeltaNet(config)" of the Evolving Transformer
 * page names the short convolution for local context and the key normalisation).
 *
 *   mixed_qkv     [total_tokens][C] bf16 with C = 2*h_qk*d_k + h_v*d_v, channels ordered
 *                 q heads | k heads | v heads, each head's d channels contiguous
 *   conv_weight   [C][conv_kernel] fp32; tap conv_kernel-1 multiplies the current token,
 *                 tap i the token conv_kernel-1-i positions earlier. No bias. The window
 *                 never reaches across a sequence start (zero history).
 *   q, k          [total_tokens][h_qk][d_k] bf16: silu(y) / max(||silu(y)||_2, 1e-12),
 *                 q further multiplied by q_scale
 *   v             [total_tokens][h_v][d_v] bf16: silu(y)
 * conv_kernel must be between 1 and 4.
 */
gdn_status gdn_conv_prep(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                         int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float q_scale,
                         void* q, void* k, void* v, void* stream);

/*
 * Front end at decode time: the short causal convolution of section "01 .
 * GatedDeltaNet(config)" of the Evolving Transformer page (with gdn_conv_prep's SiLU and
 * q/k normalisation) at one new token for each of num_seqs sequences, the inputs the
 * convolution still needs from earlier tokens kept in a window pool. Every output equals
 * what gdn_conv_prep gives for that token when run over the sequence so far (same
 * arithmetic, bit for bit), so a prompt prefilled and then decoded token by token matches
 * one prefill over the whole text.
 *
 *   mixed_qkv     [num_seqs][C] bf16, this step's projected inputs (C and channel order as
 *                 for gdn_conv_prep)
 *   conv_weight   [C][conv_kernel] fp32, as for gdn_conv_prep
 *   conv_window   [pool_size][conv_kernel-1][C] bf16, read and written in place: row r of a
 *                 slot holds the input conv_kernel-1-r tokens back (zeros for a new
 *                 sequence). After the call it holds the window for the next token. May be
 *                 NULL when conv_kernel is 1.
 *   window_slots  [num_seqs] int32: sequence n uses slot window_slots[n]; NULL means slot n.
 *                 Slots must be distinct.
 *   q, k, v       [num_seqs][h_qk][d_k], [num_seqs][h_qk][d_k], [num_seqs][h_v][d_v] bf16,
 *                 the inputs of gdn_decode_step
 */
gdn_status gdn_conv_decode_step(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                                void* conv_window, const int32_t* window_slots, int32_t num_seqs,
                                int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float q_scale,
                                void* q, void* k, void* v, void* stream);

/*
 * gdn_conv_decode_step followed by gdn_decode_step, in one launch: the front end of section
 * "01 . GatedDeltaNet(config)" of the Evolving Transformer page at one new token per
 * sequence, then one step of the rule of section "Correcting a memory instead of adding to
 * it" of page "Qwen3-Next -- How a running memory and a searchable history cooperate", with
 * the front end's q, k and v kept on chip. Outputs, the state pool and the window pool are
 * bit for bit those of the two calls; q, k and v are not written out.
 *
 *   mixed_qkv, conv_weight, conv_kernel, conv_window, window_slots, q_scale
 *                 as for gdn_conv_decode_step
 *   g, beta, state_pool, state_slots, scale, o
 *                 as for gdn_decode_step (bf16 output)
 * h_v / h_qk must be 1 or 2 (one workgroup covers the V heads of a QK head, so the shared q
 * and k channels of the window are read and shifted once); GDN_ERR_UNSUPPORTED otherwise.
 */
gdn_status gdn_decode_step_with_conv(const void* mixed_qkv, const float* conv_weight,
                                     int32_t conv_kernel, void* conv_window,
                                     const int32_t* window_slots, float q_scale, const float* g,
                                     const float* beta, float* state_pool,
                                     const int32_t* state_slots, int32_t num_seqs, int32_t h_qk,
                                     int32_t h_v, int32_t d_k, int32_t d_v, float scale, void* o,
                                     void* stream);

/*
 * The window a prefill leaves for gdn_conv_decode_step: for each sequence n of the packed
 * batch (cu_seqlens as for gdn_conv_prep), its last conv_kernel-1 inputs from mixed_qkv,
 * with zeros for positions before the sequence start, written to slot window_slots[n]
 * (NULL: slot n) of conv_window. A no-op for conv_kernel 1.
 */
gdn_status gdn_conv_window_from_prefill(const void* mixed_qkv, int32_t conv_kernel,
                                        const int32_t* cu_seqlens, int32_t num_seqs,
                                        int32_t total_tokens, int32_t h_qk, int32_t h_v,
                                        int32_t d_k, int32_t d_v, void* conv_window,
                                        const int32_t* window_slots, void* stream);

/* Output gate function of gdn_gated_rmsnorm. */
typedef enum {
    GDN_GATE_SIGMOID = 0,     /* sigmoid(z) */
    GDN_GATE_SILU = 1         /* z * sigmoid(z) */
} gdn_gate;

/*
 * Output epilogue after the mixer. The architecture knowledge-base page "Qwen3-Next
 * 80B-A3B" names the model's norm in its "Architecture" table (row "Norm type") as a
 * zero-centred RMSNorm, and section "01 . GatedDeltaNet(config)" of page "Qwen3-Next
 * 80B-A3B -- The Evolving Transformer" says a gate decides how much of the recurrent
 * read-out reaches the output. Neither gives a formula; this computes, for every token row
 * r and V head h, with x = o[r][h][:] and the gate input z[r][h][:],
 *
 *     out = x / sqrt(mean(x^2) + eps) * (1 + weight) * gate(z)     (elementwise)
 *
 * i.e. the norm over one head's d_v channels with the zero-centred scale, then the gate.
 *
 *   o, z, out   [rows][h_v][d_v] in io_dtype (GDN_BF16 or GDN_F32); out may be o or z
 *               itself (in place); other overlaps are not allowed
 *   weight      [d_v] fp32, shared by the heads (0 means a scale of 1)
 *   eps         finite and >= 0
 *   gate        GDN_GATE_SIGMOID or GDN_GATE_SILU
 * d_v must be 128; arithmetic in fp32, bf16 outputs rounded to nearest even.
 * GDN_ERR_SHAPE for negative rows, h_v < 1 or a bad eps; GDN_ERR_UNSUPPORTED for another
 * d_v, dtype or gate, or more than 2^34 vectors; GDN_ERR_NULL for a missing pointer when
 * rows > 0. rows = 0 does nothing.
 */
gdn_status gdn_gated_rmsnorm(const void* o, const void* z, gdn_dtype io_dtype, const float* weight,
                             int32_t rows, int32_t h_v, int32_t d_v, float eps, gdn_gate gate,
                             void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
