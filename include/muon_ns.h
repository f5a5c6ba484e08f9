/*
 * muon_ns.h -- C ABI of libmuon_ns.so: batched Newton-Schulz orthogonalization of Muon
 * momentum matrices (standard iteration on X and the Gram reformulation on R = X X^T)
 * and the fused Muon step, on one AMD MI355X (gfx950).
 *
 * Sources (web pages):
 *  - "Moonlight 16B Guide: Scalable MoE & Muon Optimizer", sections "The Scalable Muon
 *    Optimizer: Theory and Mechanics" (momentum -> Newton-Schulz -> update scale ->
 *    decoupled weight decay), "The Newton-Schulz Iteration for Matrix Orthogonalization",
 *    "Innovation 1", "Innovation 2" and "End-to-End PyTorch Implementation".
 *  - Jiqizhixin article on Gram Newton-Schulz: standard Newton-Schulz and its three
 *    products, the Gram reformulation, the naive variant's fp16 instability and the
 *    stabilized variant (restart after step 2, re-formed Gram matrix).
 *
 * Conventions shared by every entry point
 *  - All matrix buffers are device pointers owned by the caller. The library never
 *    allocates or frees device memory in a call; scratch space comes from the caller's
 *    workspace (size from mns_workspace_bytes).
 *  - A batch is `batch` row-major matrices of rows x cols: element (b, i, j) lives at
 *    ptr + b*stride + i*ld + j (in elements). ld >= cols; stride >= rows*ld when batch > 1.
 *  - Each matrix is orthogonalized as n x m with n = min(rows, cols), m = max(rows, cols):
 *    a matrix with rows > cols is processed as its transpose and written back transposed
 *    (no copy is asked of the caller).
 *  - Calls are asynchronous: they validate, enqueue kernels on `stream` (a hipStream_t;
 *    NULL = the null stream) and return. No host synchronisation happens inside a call.
 *    A call enqueues kernel launches only (no memset, copy or event record unless timing
 *    is switched on), so with a caller-supplied workspace it can be captured into a HIP
 *    graph and replayed.
 *  - Argument errors are returned synchronously before any HIP call, and then nothing is
 *    enqueued. A failed launch returns MNS_ERR_HIP (detail: mns_last_hip_error()).
 *  - Numerical conditions are reported per matrix in `flags` (device int32 [batch], may be
 *    NULL), written asynchronously: bit0 = the Frobenius norm is not finite, bit1 = the
 *    norm is zero (the output is then exactly zero), bit2 = a non-finite output value.
 *  - Calls that share a workspace must be ordered on one stream; calls on different
 *    streams need different workspaces.
 *  - Size limit: one n x m iterate (m rounded up to a multiple of 8, in the wider of the
 *    input and iterate dtypes) must span at most 2^31 bytes, e.g. 32768 x 32768 in bf16;
 *    larger matrices return MNS_ERR_SHAPE.
 */
#ifndef MUON_NS_H
#define MUON_NS_H

#include <stddef.h>
#include <stdint.h>

/* Exported entry points (the library is built with hidden default visibility). */
#ifndef MNS_API
#define MNS_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MNS_F32 = 0, MNS_BF16 = 1, MNS_F16 = 2 } mns_dtype;

typedef enum { MNS_VARIANT_STANDARD = 0, MNS_VARIANT_GRAM = 1 } mns_variant;

enum {
  MNS_OK = 0,
  MNS_ERR_ARG = -1,         /* null pointer, bad scalar, overlapping in/out */
  MNS_ERR_DTYPE = -2,       /* unsupported dtype or dtype combination */
  MNS_ERR_SHAPE = -3,       /* rows/cols/batch < 1, ld < cols, stride too small, shape mismatch */
  MNS_ERR_WORKSPACE = -4,   /* workspace pointer NULL or smaller than one matrix needs */
  MNS_ERR_HIP = -5,         /* a HIP call failed; see mns_last_hip_error() */
  MNS_ERR_UNSUPPORTED = -6  /* valid request the library does not implement */
};

/* A strided batch of row-major matrices (see conventions above). dtype is an mns_dtype. */
typedef struct mns_tensor {
  void* ptr;
  int32_t dtype;
  int64_t batch, rows, cols;
  int64_t ld;
  int64_t stride;
} mns_tensor;

/*
 * Newton-Schulz parameters.
 *  steps        K >= 1 (at most 64).
 *  coeffs       host pointer to K triples (a_k, b_k, c_k), row-major [K][3]: step k maps
 *               X -> a_k X + b_k (X X^T) X + c_k (X X^T)^2 X, i.e. each singular value
 *               s -> a_k s + b_k s^3 + c_k s^5. NULL = (3.4445, -4.7750, 2.0315) every step.
 *               The guide's cubic 0.5 X (3I - X^T X) is (1.5, -0.5, 0).
 *  eps          added to the Frobenius norm: X0 = G / (||G||_F + eps) (guide's listing: 1e-7).
 *  iter_dtype   storage dtype of the normalised iterates: the n x n matrices (Gram R, Z, RZ,
 *               Q; standard A = X X^T and B) and every X_k after the first step or restart.
 *               The caller's input and output keep their own dtype; accumulation is always
 *               fp32. With fp32 input it must be MNS_F32; with bf16/fp16 input it may be
 *               MNS_F16 (the usual choice: 3 more mantissa bits, and every normalised
 *               iterate is bounded well inside fp16's range) or MNS_BF16.
 *  restart_mask Gram variant only: bit k (k = 1..K-1) set = after step k form X_k = Q_k X
 *               explicitly, re-form R = X_k X_k^T and restart Q = I (the article's stabilized
 *               variant is 1u << 2; 0 is the naive variant). Bits >= K are ignored.
 */
typedef struct mns_ns_params {
  int32_t steps;
  const float* coeffs;
  float eps;
  int32_t iter_dtype;
  uint32_t restart_mask;
} mns_ns_params;

/*
 * Muon step parameters (guide, "The Scalable Muon Optimizer" box and PyTorch listing).
 *  lr, momentum (mu), weight_decay (lambda), scale_coeff: the update is
 *  U = scale_coeff * sqrt(max(rows, cols)) * NS(N) and W <- (1 - lr*lambda) W - lr U.
 *  nesterov: 0 -> N = M_t; 1 -> N = mu M_t + (1 - mu) G_t.
 *  variant: MNS_VARIANT_STANDARD or MNS_VARIANT_GRAM.
 */
typedef struct mns_step_params {
  float lr;
  float momentum;
  float weight_decay;
  float scale_coeff;
  int32_t nesterov;
  int32_t variant;
} mns_step_params;

/*
 * Workspace bytes needed to process G's batch with the given variant, in chunks of at
 * most max_batch_chunk matrices (<= 0: the whole batch in one chunk). Any workspace at
 * least as large as the max_batch_chunk = 1 figure is accepted by the calls below; they
 * then process the batch in the largest chunks that fit. Host-only; no HIP call.
 * Returns MNS_OK and *bytes, or an argument error.
 */
MNS_API int mns_workspace_bytes(int variant, const mns_tensor* G, const mns_ns_params* p,
                        int64_t max_batch_chunk, size_t* bytes);

/*
 * Standard Newton-Schulz (Jiqizhixin article, standard iteration; guide's listing):
 * X0 = G/(||G||_F + eps); for k = 1..K: A = X X^T, B = b_k A + c_k A^2, X <- a_k X + B X.
 * G: input batch (F32, BF16 or F16). O: output, same batch/rows/cols/dtype as G, must not
 * overlap G. ws/ws_bytes: device workspace. flags: device int32 [batch] or NULL.
 */
MNS_API int muon_ns_batched(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream);

/*
 * Gram Newton-Schulz (Jiqizhixin article, Gram reformulation and stabilized variant):
 * R = X0 X0^T, Q = I; for k = 1..K: Z = a_k I + b_k R + c_k R^2, Q <- Z Q, then either a
 * restart (X <- Q X, R <- X X^T, Q <- I; when bit k of restart_mask is set and k < K) or
 * R <- Z R Z (when k < K); the output is Q X. Equal to muon_ns_batched in exact arithmetic.
 * Arguments as for muon_ns_batched.
 */
MNS_API int gram_ns_batched(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream);

/*
 * One fused Muon step per matrix (guide, "The Scalable Muon Optimizer" box):
 *   M <- mu M + (1 - mu) G;  N = nesterov ? mu M + (1 - mu) G : M;
 *   O = NS(N) (sp->variant);  U = scale_coeff * sqrt(max(rows, cols)) * O;
 *   W <- (1 - lr * weight_decay) W - lr U.
 * W: weights (F32/BF16/F16), updated in place. G: gradient (same dtype as the NS input,
 * F32/BF16/F16). M: momentum, F32, updated in place. W, G, M share batch/rows/cols.
 * U_out: NULL, or a buffer of G's shape (F32/BF16/F16) that receives U (before lr).
 * N is stored in G's dtype before Newton-Schulz. Arguments otherwise as above.
 */
MNS_API int muon_step(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M,
              const mns_tensor* U_out, const mns_step_params* sp, const mns_ns_params* p,
              void* ws, size_t ws_bytes, int32_t* flags, void* stream);

/*
 * muon_step without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). The scratch
 * space is a static device array of MNS_NOALLOC_SCRATCH_BYTES compiled into the library; each
 * GPU the library runs on holds its own copy from the library's first use on that GPU until
 * the process ends. The batch is processed in the largest chunks whose workspace fits it (as
 * muon_step does with a workspace of that size, which gives identical results). The call
 * allocates and frees nothing.
 * Arguments and results as for muon_step, without ws / ws_bytes.
 * Errors: as for muon_step, and MNS_ERR_WORKSPACE when one matrix alone needs more scratch
 * than MNS_NOALLOC_SCRATCH_BYTES (returned before any HIP call; e.g. a 2048 x 7168 matrix
 * needs ~100 MB with stabilized Gram NS, a 7168 x 18432 one ~1 GB). The first call on a GPU
 * looks up that GPU's copy of the array (MNS_ERR_HIP if the lookup fails).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several threads without ordering) race on it and must not be
 * issued; calls ordered on one stream are safe. No part of the array needs to start zeroed.
 */
#define MNS_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
MNS_API int muon_step_noalloc(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M,
                      const mns_tensor* U_out, const mns_step_params* sp, const mns_ns_params* p,
                      int32_t* flags, void* stream);

/*
 * Grouped calls: ngroups (1 .. 4) strided batches of different shapes in one call, e.g. the
 * Kimi-K2 optimizer step of the Gram Newton-Schulz article's timing (expert up/gate matrices,
 * expert down matrices in the transposed orientation, and the dense FFN matrices). Every group
 * follows the conventions above on its own; all groups share one input dtype and one set of
 * parameters. When the workspace holds every group at once (mns_workspace_bytes_grouped), each
 * product step is a single launch over the tiles of all groups, so large groups' tail tiles
 * share the chip with the other groups' tiles; otherwise the groups run one after another,
 * each chunked as in the single-group calls. Results equal those of separate single-group
 * calls bit for bit.
 *  G, O, W, M, U_out: arrays of ngroups tensors (U_out may be NULL: no update output).
 *  flags: device int32 [sum of the groups' batch sizes] or NULL; group g's matrices follow
 *         those of groups 0 .. g-1.
 *  Errors as for the single-group calls, plus MNS_ERR_ARG for ngroups outside 1 .. 4 or any
 *  two output buffers (or an output and an input) that overlap.
 */
MNS_API int mns_workspace_bytes_grouped(int variant, int ngroups, const mns_tensor* G,
                                const mns_ns_params* p, size_t* bytes);
MNS_API int muon_ns_grouped(int ngroups, const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream);
MNS_API int gram_ns_grouped(int ngroups, const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream);
MNS_API int muon_step_grouped(int ngroups, const mns_tensor* W, const mns_tensor* G, const mns_tensor* M,
                      const mns_tensor* U_out, const mns_step_params* sp, const mns_ns_params* p,
                      void* ws, size_t ws_bytes, int32_t* flags, void* stream);

/*
 * AdamW for the parameters that stay off Muon (guide, "The Hybrid Optimization Strategy":
 * RMSNorm scales, biases, router projections, token embeddings; update from "The
 * Coordinate-Wise Limitation of AdamW"):
 *   m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2;
 *   p <- (1 - lr weight_decay) p - lr m^ / (sqrt(v^) + eps),
 * with m^ = m, v^ = v, or with bias_correction set m^ = m / (1 - beta1^step),
 * v^ = v / (1 - beta2^step). eps is outside the square root, as in the guide's equation.
 */
typedef struct mns_adamw_params {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t step;             /* >= 1 (used by the bias correction only) */
  int32_t bias_correction;  /* 0 or 1 */
} mns_adamw_params;

/*
 * One AdamW step over ntensors flat, contiguous tensors (host arrays of device pointers):
 * params[i] and grads[i] of `dtype` (F32, BF16 or F16; the same for all), exp_avg[i] and
 * exp_avg_sq[i] fp32, all numels[i] elements long (0 allowed). params and both moments are
 * updated in place; no two buffers may overlap. Tensors are processed 48 per launch.
 * Errors: MNS_ERR_ARG (null pointer, numel < 0, non-finite or out-of-range hyper-parameter,
 * beta outside [0, 1), overlap), MNS_ERR_DTYPE, MNS_ERR_HIP.
 */
MNS_API int adamw_step(int ntensors, void* const* params, const void* const* grads, float* const* exp_avg,
               float* const* exp_avg_sq, const int64_t* numels, int32_t dtype,
               const mns_adamw_params* ap, void* stream);

/*
 * Debug trace of the Gram iteration for the first matrix of G (diagnostics of the fp16
 * instability the Gram Newton-Schulz article describes: negative eigenvalues of the Gram
 * matrix). Runs gram_ns_batched on matrix 0 only and, after each step k = 1 .. K-1, copies the
 * Gram iterate then in use (R_k = X_k X_k^T, re-formed at restarts) into trace[k-1] as fp32.
 * trace: device float [K-1][n][n] row-major, n = min(rows, cols). O: as in gram_ns_batched
 * (only matrix 0 is written). ws: workspace for a batch of one. Requires K >= 2.
 */
MNS_API int gram_ns_trace(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p, void* ws,
                   size_t ws_bytes, float* trace, void* stream);

/* Static English text for a status code (never NULL). */
MNS_API const char* mns_status_string(int code);

/* The hipError_t of the last HIP failure on the calling thread (0 if none). */
MNS_API int mns_last_hip_error(void);

/* ABI version of this library (major * 10000 + minor * 100 + patch). */
MNS_API int mns_version(void);

/*
 * Per-kernel-kind launch timing with HIP events recorded on the call's stream around each
 * launch of the library's kernels. Off by default; when on, each launch records two events.
 *  mns_timing_enable(1/0)          switch recording on/off (host state, process-wide).
 *  mns_timing_reset()              drop recorded events.
 *  mns_timing_query(kind, ms, n)   synchronises the recorded events of `kind` and returns
 *                                  the summed duration in ms and the launch count.
 *  mns_timing_kinds()              number of kinds; kinds are 0..mns_timing_kinds()-1.
 *  mns_kernel_kind_name(kind)      static name of a kind ("gemm_rect", ...), or NULL.
 * The query returns MNS_ERR_ARG for an unknown kind and MNS_ERR_HIP on an event failure.
 */
MNS_API int mns_timing_enable(int on);
MNS_API int mns_timing_reset(void);
MNS_API int mns_timing_query(int kind, double* total_ms, int64_t* launches);
MNS_API int mns_timing_kinds(void);
MNS_API const char* mns_kernel_kind_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* MUON_NS_H */
