/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library: the
 * forward (prefill, packed prefill, decode, multi-token recurrence, each also
 * for Gated DeltaNet gates and with optional in-kernel input transforms) and
 * its backward (kda_backward).
 *
 * The operation (one head; S is d_k x d_v, row = key channel, column = value
 * channel; g = log alpha with natural log, g <= 0):
 *
 *   Sbar_t = Diag(exp(g_t)) S_{t-1}
 *   S_t    = Sbar_t + beta_t k_t (v_t - Sbar_t^T k_t)^T
 *   o_t    = S_t^T (scale * q_t)
 *
 * Definition: "Kimi Unveils Delta Attention and K3 Architecture Updates",
 * section 4 (Kimi Delta Attention: forget each key channel, predict, correct,
 * write, read) with its key-by-value reference layout, and "Kimi Delta
 * Attention: Channel-Wise Memory Control", section "Change one piece of Gated
 * DeltaNet" (S in R^{d_k x d_v}, decay by left multiplication).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer on the current HIP device, unless stated.
 *  - All arrays are dense, row-major, contiguous, with no padding.  Each
 *    array starts on a 16-byte boundary (beta and cu_seqlens: 4 bytes), as
 *    every device allocation does; otherwise KDA_ERR_ALIGN.
 *  - q, k, v, out use io_dtype (KDA_IO_F32 = float, KDA_IO_BF16 = bfloat16
 *    bit patterns); log_alpha, beta and every state are float (fp32).
 *  - The state is always fp32 and is kept fp32 on chip across a whole call.
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace.  The library allocates nothing, never frees, never
 *    synchronises the device and keeps no state between calls (except the
 *    static scratch array of kda_backward_noalloc and its per-device
 *    address, below); work is
 *    enqueued on `stream` (a hipStream_t cast to void*, NULL = the default
 *    stream) and results are valid once that stream has reached them.
 *  - Aliasing: S0 == S_final is allowed (in-place state update); any other
 *    overlap between an output and another argument is not.
 *  - Supported sizes: d_k and d_v in {64, 128}; chunk == 64.  The two
 *    prefill calls take KDA_IO_F32 only with d_k == d_v == 64 (their fp32
 *    operand tiles do not fit in LDS otherwise); decode, the recurrent calls
 *    and the backward take both types at every supported size.  Anything
 *    else returns KDA_ERR_UNSUPPORTED.
 *  - Errors: every argument is validated before any work is enqueued; on a
 *    validation error nothing is enqueued and a negative KDA_ERR_* code is
 *    returned.  KDA_ERR_HIP reports a launch failure (hipGetLastError).
 *    Values are not checked: NaN/Inf propagate; beta outside [0, 1], g > 0 or
 *    non-normalised keys give the recurrence's (possibly unstable) result.
 *  - T == 0 (or an empty packed sequence) copies S0 to S_final (zeros if S0 is
 *    NULL) and writes no output row.
 *  - Thread safety: calls are re-entrant; calls on different streams may run
 *    concurrently as long as their buffers do not overlap.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kda_io_dtype { KDA_IO_F32 = 0, KDA_IO_BF16 = 1 };

enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL */
  KDA_ERR_DIM = -2,         /* a size is negative or inconsistent */
  KDA_ERR_UNSUPPORTED = -3, /* d_k, d_v, chunk or io_dtype not supported */
  KDA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  KDA_ERR_HIP = -5,         /* a HIP launch failed */
  KDA_ERR_ALIAS = -6,       /* an output overlaps an input (other than S0 == S_final) */
  KDA_ERR_ALIGN = -7,       /* an array is not aligned (16 bytes; beta and cu_seqlens 4) */
  KDA_ERR_SCRATCH = -8      /* kda_backward_noalloc: the problem needs more scratch than
                               KDA_NOALLOC_SCRATCH_BYTES */
};

/*
 * kda_chunk_fwd -- chunkwise prefill over a batch of equal-length sequences.
 *
 * Computes exactly the recurrence above for every (b, h), scheduled chunk by
 * chunk as in "Kimi Unveils Delta Attention and K3 Architecture Updates",
 * section 6 (Chunkwise KDA): chunk-local cumulative decay, the causal
 * key-key system resolved by a unit-lower-triangular inverse, the
 * fast-forwarded state and the causal outputs.  A last partial chunk behaves
 * as if padded with tokens that leave the state unchanged.
 *
 *  q, k       [B, T, H, d_k]  io_dtype
 *  v          [B, T, H, d_v]  io_dtype
 *  log_alpha  [B, T, H, d_k]  fp32, g = log alpha (natural log)
 *  beta       [B, T, H]       fp32
 *  S0         [B, H, d_k, d_v] fp32, or NULL for a zero initial state
 *  out        [B, T, H, d_v]  io_dtype (bf16 results are rounded to nearest even)
 *  S_final    [B, H, d_k, d_v] fp32, or NULL to skip
 *  scale      multiplies q (the pages' default is d_k^-1/2)
 *  chunk      tokens per chunk; must be 64
 *  workspace  device scratch of at least kda_chunk_fwd_workspace_size(...)
 *             bytes, 256-byte aligned, overlapping no other argument.  It is
 *             required when the call takes the chunk-parallel schedule (bf16,
 *             d_k = d_v = 128, plain KDA gates, at most 64 chains of at least
 *             512 tokens: KDA_ERR_WORKSPACE without it), which forms the WY
 *             factors of every chunk at once into the workspace and then scans
 *             each chain's state over them ("Kimi Unveils Delta Attention and
 *             K3 Architecture Updates", section 6.6).  Otherwise it may be
 *             NULL; given, it enables the balanced schedule described under
 *             kda_chunk_fwd_varlen (the B sequences of T tokens laid end to
 *             end) for calls of one to four times as many chains as the GPU
 *             runs at once, with bit-identical results.  Its contents need no
 *             initialisation; calls that share it must be ordered on one
 *             stream.
 * Returns KDA_OK or a KDA_ERR_* code.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                  const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                  int H, int d_k, int d_v, float scale, int chunk, int io_dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_varlen -- chunkwise prefill over N packed variable-length
 * sequences.  Sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]) of the
 * packed token axis; its state starts from S0[n] and never crosses into
 * another sequence ("Linear Attention, From Scratch to Kimi 3", section 9,
 * cu_seqlens).  Chunks never straddle two sequences.
 *
 *  q, k       [T_total, H, d_k]  io_dtype
 *  v, out     [T_total, H, d_v]  io_dtype
 *  log_alpha  [T_total, H, d_k]  fp32
 *  beta       [T_total, H]       fp32
 *  S0         [N, H, d_k, d_v]   fp32 or NULL (zeros)
 *  S_final    [N, H, d_k, d_v]   fp32 or NULL
 *  cu_seqlens [N + 1] int32, DEVICE memory: cu_seqlens[0] == 0,
 *             non-decreasing, cu_seqlens[N] == T_total.  These preconditions
 *             are not checked on the device (the values are never read on the
 *             host); a violation gives undefined results.
 *  workspace  NULL, or device memory of at least
 *             kda_chunk_fwd_varlen_workspace_size(...) bytes, 256-byte
 *             aligned, overlapping no other argument (else KDA_ERR_WORKSPACE,
 *             KDA_ERR_ALIGN, KDA_ERR_ALIAS).  Its contents need no
 *             initialisation.  With a workspace, a call of few long sequences
 *             (bf16, d_k = d_v = 128, plain KDA gates, at most 64 chains, at
 *             least 512 tokens per sequence on average) takes the
 *             chunk-parallel schedule described under kda_chunk_fwd, with
 *             its records listed per sequence (results within rounding of
 *             the schedule without a workspace); and a call of more (sequence,
 *             head) chains than the GPU runs at once (and at most four times
 *             as many) balances the chunks over the resident workgroups:
 *             sequences are laid end to end and cut into equal slices
 *             (McNaughton's wrap-around rule), a sequence that crosses a cut
 *             continues on the next workgroup from the fp32 state handed over
 *             in the workspace.  Chunks stay aligned to their sequence, so
 *             the results are bit-identical to those without a workspace.
 *             Calls that share a workspace must be ordered on one stream.
 *             A workgroup waits for a handed-over state for a bounded number
 *             of polls (2^22, or the count in the environment variable
 *             KDA_SPLIT_SPIN_POLLS, read on every call) and past it
 *             recomputes the sequence's first chunks itself: same results,
 *             more work (tests set 0 to take that path).
 * Returns KDA_OK or a KDA_ERR_* code.
 */
int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, void* out, float* S_final,
                         const int32_t* cu_seqlens, int N, int T_total, int H, int d_k, int d_v,
                         float scale, int chunk, int io_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_decode_step -- one token for each of N sequences: the fused recurrent
 * step ("Kimi Unveils Delta Attention and K3 Architecture Updates", section 5:
 * decay, prediction reduction, outer-product write, read reduction).  Each
 * head's fp32 state is read once and written once.
 *
 *  q, k       [N, H, d_k]  io_dtype
 *  v, out     [N, H, d_v]  io_dtype
 *  log_alpha  [N, H, d_k]  fp32
 *  beta       [N, H]       fp32
 *  S_inout    [N, H, d_k, d_v] fp32, updated in place
 * Returns KDA_OK or a KDA_ERR_* code.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, float* S_inout, void* out, int N, int H, int d_k, int d_v,
                    float scale, int io_dtype, void* stream);

/*
 * kda_recurrent_fwd -- the recurrence itself, token by token, for B sequences
 * of T tokens each: multi-token decode, speculative verification, short
 * prefill ("Kimi Unveils Delta Attention and K3 Architecture Updates",
 * section 5, the fused recurrent kernel, which suits short sequences and
 * stateful serving; "Linear Attention, From Scratch to Kimi 3", section 9: the
 * fused kernel can loop over several tokens).  Each head's fp32 state is read
 * once from S0 and written
 * once to S_final whatever T is; the serial work grows with T, so for long
 * sequences kda_chunk_fwd is the faster schedule of the same result.
 *
 *  q, k       [B, T, H, d_k]  io_dtype
 *  v, out     [B, T, H, d_v]  io_dtype
 *  log_alpha  [B, T, H, d_k]  fp32
 *  beta       [B, T, H]       fp32
 *  S0         [B, H, d_k, d_v] fp32 or NULL (zeros)
 *  S_final    [B, H, d_k, d_v] fp32 or NULL; S_final == S0 updates the state
 *             in place (the usual serving call)
 *  d_k, d_v in {64, 128}; both io_dtype values for every shape.
 * Returns KDA_OK or a KDA_ERR_* code.
 */
int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                      int H, int d_k, int d_v, float scale, int io_dtype, void* stream);

/*
 * kda_recurrent_fwd_varlen -- kda_recurrent_fwd over N packed sequences of
 * any lengths (zero included): sequence n owns tokens [cu_seqlens[n],
 * cu_seqlens[n+1]) and state slot n ("Linear Attention, From Scratch to Kimi
 * 3", section 9, cu_seqlens).  Layouts and cu_seqlens preconditions as for
 * kda_chunk_fwd_varlen; S0 == S_final allowed.
 * Returns KDA_OK or a KDA_ERR_* code.
 */
int kda_recurrent_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, void* out, float* S_final,
                             const int32_t* cu_seqlens, int N, int T_total, int H, int d_k,
                             int d_v, float scale, int io_dtype, void* stream);

/*
 * Gated DeltaNet through the same calls: one forget gate per (token, head),
 * shared by every key channel ("Kimi Unveils Delta Attention and K3
 * Architecture Updates", section 3; "Linear Attention, From Scratch to Kimi
 * 3", section 5).  The recurrence above with g_t[i] = g_t for every key
 * channel i, i.e. S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t
 * v_t^T.  Each kda_gdn_* call takes exactly the arguments of its kda_*
 * counterpart, except that log_alpha has no d_k axis:
 *
 *  kda_gdn_chunk_fwd, kda_gdn_recurrent_fwd   log_alpha [B, T, H]      fp32
 *  kda_gdn_chunk_fwd_varlen,
 *  kda_gdn_recurrent_fwd_varlen                log_alpha [T_total, H]   fp32
 *  kda_gdn_decode_step                         log_alpha [N, H]         fp32
 *
 * log_alpha needs 4-byte alignment only.  Same sizes, dtypes, aliasing rules
 * and status codes as the KDA calls.
 */
int kda_gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                      int H, int d_k, int d_v, float scale, int chunk, int io_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);
int kda_gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, void* out, float* S_final,
                             const int32_t* cu_seqlens, int N, int T_total, int H, int d_k,
                             int d_v, float scale, int chunk, int io_dtype, void* workspace,
                             size_t workspace_bytes, void* stream);
int kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, float* S_inout, void* out, int N, int H, int d_k,
                        int d_v, float scale, int io_dtype, void* stream);
int kda_gdn_recurrent_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* S0, void* out, float* S_final, int B,
                          int T, int H, int d_k, int d_v, float scale, int io_dtype,
                          void* stream);
int kda_gdn_recurrent_fwd_varlen(const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const float* S0,
                                 void* out, float* S_final, const int32_t* cu_seqlens, int N,
                                 int T_total, int H, int d_k, int d_v, float scale, int io_dtype,
                                 void* stream);

/*
 * Input transforms applied inside the kernels to each token's raw inputs,
 * before the step ("Linear Attention, From Scratch to Kimi 3", sections 6 and
 * 7, the layer around the recurrence), so that no separate pass over q, k,
 * log_alpha or beta is needed:
 *
 *  KDA_PRO_QK_L2NORM     q <- q / sqrt(sum q^2 + 1e-6), likewise k, per
 *                        (token, head) vector, in fp32 (section 7: each head's
 *                        q and k are L2-normalised)
 *  KDA_PRO_BETA_SIGMOID  beta holds logits: beta <- 1 / (1 + exp(-beta))
 *                        (section 6: a sigmoid applied inside the kernel)
 *  KDA_PRO_GATE          log_alpha holds the raw gate projection g:
 *                        log alpha = -5 sigmoid(exp(A_log[h]) (g + gate_bias))
 *                        (section 6: -5 times a sigmoid, a log-retention in
 *                        (-5, 0), from the projection, a learned per-channel
 *                        bias and one learned sensitivity per head; the page's
 *                        formula is lost, and this composition inside the
 *                        sigmoid is this library's reading of the text)
 *
 * A_log is [H] fp32 (required with KDA_PRO_GATE); gate_bias is [H, d_k] fp32,
 * or [H] with per-head gates, or NULL for zero.  Both 4-byte aligned, device
 * memory, not overlapping any output.  Unknown flag bits return
 * KDA_ERR_UNSUPPORTED.
 */
#define KDA_PRO_QK_L2NORM 1u
#define KDA_PRO_BETA_SIGMOID 2u
#define KDA_PRO_GATE 4u

typedef struct kda_prologue {
  uint32_t flags;          /* KDA_PRO_* bits */
  const float* A_log;      /* [H] */
  const float* gate_bias;  /* [H, d_k], [H] (per-head gates) or NULL */
} kda_prologue;

/*
 * The fused forms of the three operations: every variant above through one
 * entry point each, with optional input transforms.
 *
 *  cu_seqlens     NULL: N sequences of T tokens in the batched layout (as
 *                 kda_chunk_fwd / kda_recurrent_fwd); otherwise N packed
 *                 sequences with T = T_total (as the _varlen calls)
 *  per_head_gate  0: KDA (log_alpha with a d_k axis); 1: Gated DeltaNet
 *                 (log_alpha without it, as the kda_gdn_* calls)
 *  pro            the input transforms, or NULL for none (the results are
 *                 then those of the plain calls)
 * Other arguments, layouts, aliasing rules and status codes as in the plain
 * calls.
 */
int kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* S0, void* out, float* S_final,
                        const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                        float scale, int chunk, int io_dtype, int per_head_gate,
                        const kda_prologue* pro, void* workspace, size_t workspace_bytes,
                        void* stream);
int kda_recurrent_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                            float scale, int io_dtype, int per_head_gate,
                            const kda_prologue* pro, void* stream);
int kda_decode_step_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, float* S_inout, void* out, int N, int H, int d_k,
                          int d_v, float scale, int io_dtype, int per_head_gate,
                          const kda_prologue* pro, void* stream);

/*
 * kda_backward -- gradients of the forward (training).  The pages give no
 * backward; chunkwise KDA is the training form ("Kimi Unveils Delta Attention
 * and K3 Architecture Updates", section 6), so this is the reverse-mode
 * derivative of the recurrence of section 4 (forget, predict, correct, write,
 * read after the write) for L(out, S_final).
 *
 * bf16 I/O at d_k = d_v = 128 runs it in the chunkwise form of section 6 on
 * MFMA (32-token chunks: a forward sweep stores each chunk's state, then a
 * reverse sweep takes every gradient contraction as a matrix product; bf16
 * operands, fp32 accumulation and fp32 state and gradient carries).  A chain
 * with a chunk half whose log decay exceeds 76 in some key channel (log alpha
 * below about -4.7 on average over 16 tokens) is redone by the token loop.
 * Every other case runs the token loop, fp32 throughout.  Inside a workgroup
 * of the chunkwise form one wave hands each chunk's triangular-solve input to
 * another and that wave waits for it a bounded number of polls (512, or the
 * count in the environment variable KDA_BWD_SPIN_POLLS, read on every call);
 * past the bound it forms the input itself: same results, more work (tests
 * set 0 to take that path).
 *
 *  inputs     q, k, v, log_alpha, beta, S0, cu_seqlens, N, T, H, d_k, d_v,
 *             scale, io_dtype, per_head_gate: exactly as given to the forward
 *             (kda_chunk_fwd / kda_recurrent_fwd and their varlen and
 *             Gated DeltaNet forms; cu_seqlens NULL = batched layout)
 *  d_out      dL/dout, shaped like out, io_dtype
 *  dS_final   dL/dS_final [N, H, d_k, d_v] fp32, or NULL (zero)
 *  dq, dk     [rows, H, d_k] fp32                 (rows = N*T or T_total)
 *  dv         [rows, H, d_v] fp32
 *  dlog_alpha [rows, H, d_k] fp32 ([rows, H] with per_head_gate)
 *  dbeta      [rows, H] fp32
 *  dS0        dL/dS0 [N, H, d_k, d_v] fp32, or NULL (not written)
 *  workspace  device memory of at least kda_backward_workspace_size() bytes,
 *             16-byte aligned, overlapping nothing else, clobbered.  It holds
 *             one flag per chain, then either every 32-token chunk's state
 *             and triangular-solve factors in bf16 (the chunkwise form) or,
 *             for the token loop, the state at the start of every 8-token
 *             block and v - p of every token
 *
 * Every gradient is written in full (rows of empty sequences have none).  No
 * output may overlap an input, another output or the workspace.  d_k and d_v
 * are 64 or 128; io_dtype fp32 or bf16.  Status codes as the forward calls.
 */
size_t kda_backward_workspace_size(int N, int T, int H, int d_k, int d_v, int packed);
int kda_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* S0, const void* d_out, const float* dS_final,
                 float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                 const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v, float scale,
                 int io_dtype, int per_head_gate, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * kda_backward_noalloc -- kda_backward for callers that cannot allocate
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and status codes as
 * kda_backward, without the workspace: the library keeps it in a static
 * device array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) on each device it runs
 * on, held until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); the caller still passes every input and
 * output.
 *
 *  - A problem whose kda_backward_workspace_size() exceeds
 *    KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_SCRATCH (nothing enqueued).
 *    At d_k = d_v = 128 that is about 7,700 head-tokens (rows x H).
 *  - The first call on a device looks up that device's array address
 *    (hipGetSymbolAddress, with the device current); later calls reuse it.
 *  - Every call on one device shares that device's array, which keeps the
 *    last call's contents.  Calls that overlap in time on one device (other
 *    streams, other threads) race on it and give undefined results; order
 *    them on one stream.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_backward_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, const void* d_out,
                         const float* dS_final, float* dq, float* dk, float* dv,
                         float* dlog_alpha, float* dbeta, float* dS0,
                         const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                         float scale, int io_dtype, int per_head_gate, void* stream);

/* KDA_NOALLOC_SCRATCH_BYTES, as the library was built. */
size_t kda_noalloc_scratch_bytes(void);

/* Workspace bytes kda_chunk_fwd (and kda_gdn_chunk_fwd, kda_chunk_fwd_fused
 * without cu_seqlens) takes for these sizes: the chunk-parallel schedule's
 * factors for the shapes that take it, else the balanced schedule's plan and
 * hand-over states (as kda_chunk_fwd_varlen_workspace_size with N = B).  0 for
 * unsupported sizes; the arguments are not otherwise validated here. */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                    int io_dtype);

/* Workspace bytes kda_chunk_fwd_varlen (and kda_gdn_chunk_fwd_varlen,
 * kda_chunk_fwd_fused with cu_seqlens) takes: for plain KDA shapes that take
 * the chunk-parallel schedule, its chunk table and the records of at most
 * H * (ceil(T_total / 64) + N) chunks; otherwise the balanced schedule's plan
 * (per-sequence chunk prefix sums, hand-over flags) and one fp32 d_k x d_v
 * state per hand-over slot, min(N * H, 1024) slots; 0 for unsupported sizes
 * (the arguments are not otherwise validated here). */
size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v,
                                           int chunk, int io_dtype);

/* A static, human-readable name for a status code. */
const char* kda_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
