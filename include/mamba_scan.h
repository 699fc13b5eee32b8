/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Operations, all from the discrete selective state-space model:
 *
 *   mamba_scan_fwd       the whole-sequence forward ("scan") over known tokens;
 *   mamba_scan_fwd_conv  the same forward with the block's short causal convolution and SiLU
 *                        fused into the scan's load stage (u computed from x on the fly);
 *   mamba_state_update   one generation step for one new token per sequence;
 *   mamba_scan_bwd       the gradients of mamba_scan_fwd (training), recomputing the state.
 *
 * The model (sources by page title and section):
 *   - "Mamba" (elemedex dex entry), "How it works": h_t = Abar*h_{t-1} + Bbar*x_t, y_t = C*h_t,
 *     with Delta, B and C functions of the current token.
 *   - "State Spaces, Selectively -- Mamba" (papermap explainer), chapter 02 "The Discretized
 *     View": the step size Delta discretizes the continuous SSM; Abar and Bbar derive from
 *     (Delta, A, B); the hardware-aware scan never materializes the expanded state in HBM, and
 *     generation is a pure recurrence with O(1) work per token.
 *   - "Mamba" (visual-learn), "Training without stepping token by token": during training the
 *     whole sequence is known and the affine updates are combined as a parallel scan; during
 *     generation the state is updated one token at a time.
 *   - Per element (the rules the pages leave open, fixed here):
 *       delta  = softplus(delta_raw + delta_bias[d])   (bias optional; softplus if flag != 0)
 *       Abar_n = exp(delta * A[d,n])
 *       Bbar_n * x = delta * B[b,n,t] * u[b,d,t]
 *       h_n    = Abar_n * h_n + Bbar_n * x            (h starts at 0 for the scan)
 *       y      = sum_n C[b,n,t] * h_n + D[d] * u      (D optional; readout after the update)
 *       out    = y * silu(z[b,d,t])                   (z optional; silu(z) = z / (1 + e^-z))
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (memory the caller allocated on the current HIP
 *     device).  The caller owns every buffer; the library allocates nothing and keeps no pointer
 *     after returning.  Its only state is the fixed scratch array of mamba_scan_fwd_noalloc (one
 *     per GPU, from module load to process exit) and that array's per-device address.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the default stream)
 *     and runs asynchronously.  Buffers must stay valid until the stream reaches the work.
 *     The library never synchronizes; device faults surface at the caller's synchronization.
 *   - Arguments are validated on the host before anything is launched.  On any error nothing is
 *     launched and nothing is written; the return value is a negative MAMBA_ERR_* code.
 *   - `out` must not alias any input; `state` must not alias `out`.
 *   - Calls on different streams with different output and workspace buffers are thread-safe.
 *   - No C++ exception crosses this interface.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 4

enum mamba_status {
  MAMBA_OK = 0,
  MAMBA_ERR_NULL = -1,        /* a required pointer is NULL */
  MAMBA_ERR_SHAPE = -2,       /* a dimension is <= 0, too large, or chunk_len is invalid */
  MAMBA_ERR_DTYPE = -3,       /* io_dtype is not one of enum mamba_dtype */
  MAMBA_ERR_UNSUPPORTED = -4, /* dstate != 16, or conv_width outside 1..4 */
  MAMBA_ERR_ALIGN = -5,       /* a pointer is not aligned to its element size */
  MAMBA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the *_workspace_bytes() query */
  MAMBA_ERR_HIP = -7,         /* the HIP runtime rejected a launch or a call */
  MAMBA_ERR_SCRATCH = -8      /* mamba_scan_fwd_noalloc: the plan needs more than its scratch */
};

/* Size of the fixed scratch array behind mamba_scan_fwd_noalloc (bytes, per GPU). */
#define MAMBA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Storage type of u, delta, z, B, C and out.  A, D, delta_bias, last_state and state are
 * always fp32.  Arithmetic is always fp32; bf16 outputs are rounded to nearest, ties to even. */
enum mamba_dtype { MAMBA_F32 = 0, MAMBA_BF16 = 1 };

/* batch * dim * seqlen is at most 2^40 elements (MAMBA_ERR_SHAPE otherwise). */
typedef struct mamba_dims {
  int64_t batch;     /* number of sequences, >= 1 */
  int64_t dim;       /* channels D, >= 1 */
  int64_t dstate;    /* state size N; must be 16 */
  int64_t seqlen;    /* tokens L, >= 1 (must be 1 for mamba_state_update) */
  int32_t io_dtype;  /* enum mamba_dtype */
  int32_t chunk_len; /* scan only: 0 = chosen by the library; otherwise the sequence is split into
                        chunks of this many tokens (a positive multiple of 16) whose carries are
                        combined with the affine composition rule.  Results agree up to fp32
                        rounding for every chunk length. */
} mamba_dims;

/* Bytes of device workspace mamba_scan_fwd needs for these dims (0 when the sequence is processed
 * as a single chunk).  Returns 0 as well for invalid dims (mamba_scan_fwd reports the error). */
size_t mamba_scan_workspace_bytes(const mamba_dims* dims);

/*
 * Selective-scan forward from a zero state over `seqlen` tokens: the layer maps the whole known
 * sequence to an output of the same shape ("Mamba" (elemedex), "How it works": the discrete
 * selective SSM with Delta, B, C per token; "Mamba" (visual-learn), "Training without stepping
 * token by token": with every token known, the per-token affine updates are combined as a
 * parallel scan instead of a token-by-token loop).
 *
 *   u, delta, z, out : (batch, dim, seqlen), seqlen innermost, io_dtype
 *   B, C             : (batch, dstate, seqlen), io_dtype; shared by all channels of a sequence
 *   A                : (dim, dstate) fp32
 *   D, delta_bias    : (dim) fp32
 *   last_state       : (batch, dim, dstate) fp32; receives h after the last token
 *   workspace        : device scratch of at least mamba_scan_workspace_bytes(dims) bytes
 *                      (may be NULL when that is 0); contents on entry are ignored
 *
 * NULL allowed for D (no skip), z (no gate), delta_bias (zero bias), last_state (not written).
 * softplus_flag != 0 applies softplus to delta_raw + bias.
 * seqlen * 32 * sizeof(io element) must stay below 2^32 (seqlen < 2^25 in fp32, 2^26 in bf16;
 * MAMBA_ERR_SHAPE otherwise): a workgroup addresses its 32 channel rows with 32-bit offsets.
 * The same bound applies to every entry point that runs the forward scan (the fused-conv forward,
 * the backward's recomputation and the block).
 */
int mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag,
                   void* out, float* last_state, const mamba_dims* dims, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * mamba_scan_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * chunk records that mamba_scan_fwd keeps in the caller's workspace go to a fixed device array
 * of MAMBA_NOALLOC_SCRATCH_BYTES inside the library instead; this entry point calls no hipMalloc,
 * hipFree or allocating library routine.
 *
 *   arguments        : as for mamba_scan_fwd, minus workspace and workspace_bytes
 *
 * Returns MAMBA_ERR_SCRATCH, before anything is launched, when mamba_scan_workspace_bytes(dims)
 * exceeds MAMBA_NOALLOC_SCRATCH_BYTES (long sequences with many channels; e.g. batch*dim*(chunks-1)
 * above about 246,000 chunk records of 68 bytes).  The array of the CURRENT device is used, so
 * `stream` must belong to the current device; its address is resolved on the first call on each
 * device (MAMBA_ERR_HIP if that fails).  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (different streams, or threads without ordering) race and give
 * wrong results.  Calls on one stream are ordered and safe.  Nothing in the array has to start
 * at zero (each call writes every record before reading it); it keeps the last call's contents.
 */
int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* delta_bias,
                           int softplus_flag, void* out, float* last_state,
                           const mamba_dims* dims, void* stream);

/*
 * mamba_scan_fwd with u = silu(causal_conv1d(x)), the short depthwise convolution and SiLU that
 * precede the selective SSM in a Mamba block ("Mamba" (elemedex), "How it works"; "State Spaces,
 * Selectively -- Mamba" (papermap), ch.02: a short convolution and a nonlinearity before the
 * SSM; the width is not on the pages and is a parameter), computed inside the scan's load stage
 * so u never round-trips through HBM:
 *     u[b,d,t] = silu(conv_bias[d] + sum_{k<W} conv_weight[d,k] * x[b,d,t-(W-1)+k]),
 *     x at t < 0 is zero (causal; the newest token meets the last tap, as a cross-correlation).
 *
 *   x                : (batch, dim, seqlen), io_dtype -- replaces u of mamba_scan_fwd
 *   conv_weight      : (dim, conv_width) fp32, conv_width in 1..4 (MAMBA_ERR_UNSUPPORTED otherwise)
 *   conv_bias        : (dim) fp32 or NULL (zero)
 *   u_out            : (batch, dim, seqlen), io_dtype, or NULL: receives u (for a backward pass)
 *   everything else  : as for mamba_scan_fwd (same workspace query)
 */
int mamba_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                        int conv_width, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        int softplus_flag, void* out, float* last_state, void* u_out,
                        const mamba_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * One generation step for `batch` sequences: the state is read and updated in place and one
 * output per channel is written ("Mamba" (visual-learn), "Training without stepping token by
 * token": during generation the fixed-size state absorbs one new token at a time at the same
 * cost per token; "Mamba" (elemedex), "How it works": the same discrete update as the scan).
 *
 *   state            : (batch, dim, dstate) fp32, updated in place
 *   u, delta, z, out : (batch, dim), io_dtype
 *   B, C             : (batch, dstate), io_dtype
 *   A, D, delta_bias : as for mamba_scan_fwd
 *
 * dims->seqlen must be 1, dims->batch at most 65535 and dims->dim below 2^28 (MAMBA_ERR_SHAPE
 * otherwise);
 * dims->chunk_len is ignored.  state and A must be 16-byte aligned.  NULL allowed for D, z,
 * delta_bias.
 */
int mamba_state_update(float* state, const void* u, const void* delta, const float* A,
                       const void* B, const void* C, const float* D, const void* z,
                       const float* delta_bias, int softplus_flag, void* out,
                       const mamba_dims* dims, void* stream);

/* Bytes of device workspace mamba_scan_bwd needs for these dims (0 for invalid dims).  It holds
 * the recomputation checkpoints (64 bytes per channel and 8 tokens), the per-workgroup channel sums
 * of dB and dC (128 bytes per 32 channels and token) and small per-chunk records. */
size_t mamba_scan_bwd_workspace_bytes(const mamba_dims* dims);

/*
 * Gradients of mamba_scan_fwd (same inputs and flags) for the loss
 *     sum(out * dout) + sum(last_state * dlast),
 * sources: "State Spaces, Selectively -- Mamba" (papermap), chapters 01/02 (the scan is trained
 * with activation recomputation: the backward recomputes the expanded state instead of storing
 * it); "Mamba remembers by forgetting, read closely" (interactiveml.org), composition equation
 * (the adjoint of the affine recurrence is an affine recurrence run backwards in time, so chunks
 * compose their carries the same way).  Per element, with lam the adjoint of h:
 *     lam_t = dy_t C_t + Abar_{t+1} lam_{t+1} (lam after the last token = dlast),
 *     dy_t = dout_t silu(z_t),  dz_t = dout_t (sum_n C h_t + D u_t) silu'(z_t),
 *     ddelta_t = sigmoid(raw_t + bias) * sum_n lam_t (Abar_t A_n h_{t-1} + B_t u_t)
 *                (without softplus the sigmoid factor is 1),
 *     du_t = dy_t D + Delta_t sum_n lam_t B_t,  dA = sum_{b,t} lam_t Abar_t Delta_t h_{t-1},
 *     dB[b,n,t] = sum_d lam_t Delta_t u_t,  dC[b,n,t] = sum_d dy_t h_t,
 *     dD = sum_{b,t} dy_t u_t,  ddelta_bias = sum_{b,t} ddelta_t.
 *
 *   inputs           : as for mamba_scan_fwd (u, delta, A, B, C, D, z, delta_bias, softplus_flag)
 *   dout             : (batch, dim, seqlen), io_dtype -- gradient of out
 *   dlast            : (batch, dim, dstate) fp32 -- gradient of last_state; NULL = zero
 *   du, ddelta, dz   : (batch, dim, seqlen), io_dtype; ddelta is w.r.t. the raw delta input
 *   dB, dC           : (batch, dstate, seqlen), io_dtype
 *   dA               : (dim, dstate) fp32
 *   dD, ddelta_bias  : (dim) fp32; may be NULL (not written).  Written also when D / delta_bias is
 *                      NULL: then they are the gradients for a zero skip / zero bias.
 *   workspace        : >= mamba_scan_bwd_workspace_bytes(dims) bytes, 16-byte aligned; contents on
 *                      entry are ignored
 *
 * dz must be non-NULL when z is given and is ignored otherwise.  Every output is overwritten (not
 * accumulated).  Sums over channels, tokens and sequences are taken in a fixed order, so results
 * are bitwise reproducible for fixed dims (including chunk_len).  Arithmetic is fp32.
 */
int mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag,
                   const void* dout, const float* dlast, void* du, void* ddelta, float* dA,
                   void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                   const mamba_dims* dims, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Batched bf16 matrix product on the matrix cores, for the learned projections of a Mamba block
 * ("Mamba" (visual-learn), "Simplifications and limits": the trained layer puts linear maps around
 * the SSM;
 * "Mamba" (elemedex), "How it works": the block starts with a linear projection):
 *     C[b] (M x N) = A (M x K) * B[b] (K x N),  fp32 accumulation, bf16 output (RNE).
 *   A : row-major, element (m, k) at A[m*lda + k], lda >= K; shared by every b
 *   B : b_kcontig != 0: element (k, n) at B[b*b_bstride + n*ldb + k] (ldb >= K);
 *       b_kcontig == 0: element (k, n) at B[b*b_bstride + k*ldb + n] (ldb >= N)
 *   C : c_trans == 0: element (m, n) at C[b*c_bstride + m*ldc + n] (ldc >= N);
 *       c_trans != 0: element (m, n) at C[b*c_bstride + n*ldc + m] (ldc >= M, ldc % 4 == 0,
 *       C 8-byte aligned)
 * A, B and C hold bf16 values (16-bit storage).  Requirements (MAMBA_ERR_SHAPE / _ALIGN otherwise):
 * M % 16 == 0, N % 8 == 0, K % 8 == 0, lda and ldb multiples of 8, A and B 16-byte aligned,
 * 1 <= batch <= 65535; M, N, K, lda, ldb and ldc below 2^31, b_bstride and c_bstride in
 * [0, 2^40).  C must not overlap A or B.
 */
int mamba_gemm_bf16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                    int64_t batch, int64_t lda, int64_t ldb, int64_t b_bstride, int64_t ldc,
                    int64_t c_bstride, int b_kcontig, int c_trans, void* stream);

/* Sizes of a Mamba block (mamba_block_fwd).  seqlen, d_model, d_inner and dt_rank are at most
 * 2^30, batch * seqlen * 2 * d_inner and batch * seqlen * d_model at most 2^40, and seqlen stays
 * within the scan's bound for bf16 (seqlen < 2^26); MAMBA_ERR_SHAPE otherwise, before anything is
 * launched. */
typedef struct mamba_block_dims {
  int64_t batch;      /* sequences, 1..65535 */
  int64_t seqlen;     /* tokens L, a multiple of 8 */
  int64_t d_model;    /* width of the block's input and output, a multiple of 16 */
  int64_t d_inner;    /* channels E of the scan, a multiple of 16 */
  int64_t dstate;     /* N, must be 16 */
  int64_t dt_rank;    /* R, rank of the Delta projection, a multiple of 16 */
  int32_t conv_width; /* 1..4 */
  int32_t reserved;   /* set to 0 */
} mamba_block_dims;

/* Bytes of device workspace mamba_block_fwd needs (0 for invalid dims): the bf16 intermediates
 * x, z, u, Delta_raw, y (5 x batch*E*L), Delta_low, B, C, the fp32 split-K partials of the
 * W_x projection (when it is split) and the scan's chunk records. */
size_t mamba_block_workspace_bytes(const mamba_block_dims* dims);

/*
 * A whole Mamba block forward with caller-supplied (e.g. random) weights, sources: "Mamba"
 * (elemedex), "How it works" (linear projection, short convolution, selective SSM, multiplicative
 * gate); "State Spaces, Selectively -- Mamba" (papermap), ch.02 (Delta, B, C computed from the
 * token); "Mamba" (visual-learn), "Simplifications and limits" (trained linear maps around the
 * SSM, a brief convolution ahead of it, gating behind it).  Per sequence, with E = d_inner, R = dt_rank, N = dstate:
 *     [x; z]          = W_in hidden^T                      W_in  (2E, d_model) bf16
 *     u               = silu(causal_conv1d(x) + conv_bias)  conv_weight (E, conv_width) fp32
 *     [dlow; B; C]    = W_x u                               W_x   (R + 2N, E) bf16
 *     Delta_raw       = W_dt dlow                           W_dt  (E, R) bf16
 *     y               = scan(u, Delta_raw, A, B, C, D, z, dt_bias, softplus)   (mamba_scan_fwd)
 *     out             = (W_out y)^T                         W_out (d_model, E) bf16
 *   hidden, out : (batch, seqlen, d_model) bf16, token-major; out 8-byte aligned
 *   A           : (E, N) fp32; D, dt_bias, conv_bias: (E) fp32 or NULL (zero)
 * The projections run as bf16 MFMA GEMMs with fp32 accumulation; intermediates are stored in
 * bf16 in the workspace (>= mamba_block_workspace_bytes, 256-byte aligned).  Weight matrices and
 * hidden must be 16-byte aligned, A 16-byte aligned.
 */
int mamba_block_fwd(const void* hidden, const void* w_in, const float* conv_weight,
                    const float* conv_bias, const void* w_x, const void* w_dt,
                    const float* dt_bias, const float* A, const float* D, const void* w_out,
                    void* out, const mamba_block_dims* dims, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* mamba_status_string(int status);

/* MAMBA_SCAN_ABI_VERSION of the built library. */
int mamba_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
