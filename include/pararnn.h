/*
 * pararnn.h -- C ABI of libpararnn.so, the MI355X (gfx950) hot path of the
 * ParaRNN method: Newton solves of diagonal GRU / LSTM recurrences whose
 * linear solves are parallel scans over time, and the reverse-scan VJP.
 *
 * Method (pararnn-torch README on PyPI, section "Method"; ParaRNN abstract on
 * the HF paper list): the whole hidden trajectory H = (h_0 .. h_{T-1}) is the
 * unknown of the system  F(H)_t = h_t - f(h_{t-1}, x_t) = 0,  solved with a
 * few Newton iterations; each iteration's linearised system
 *     delta_t = J_t delta_{t-1} - r_t,   r_t = h_t - f(h_{t-1}, x_t),
 *     J_t = d f / d h (h_{t-1}, x_t)
 * is a first-order linear recurrence, solved here by a parallel scan along
 * time.  The backward pass (same page, "Method") is the adjoint: a
 * reverse linear recurrence with transposed Jacobians.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory; the library never allocates device memory (the allocation-free
 *    entry point's workspace is a static device array) and keeps no state
 *    between calls except a process-wide launch counter and, per device, the
 *    number of workgroups of a kernel that fit on it at once (queried once).
 *  - Layouts are dense and row-major: a "[B][T][D]" plane has element
 *    (b, t, d) at offset (b*T + t)*D + d, channels (d) fastest.  A state
 *    trajectory "[S][B][T][D]" holds S such planes (LSTM: plane 0 = c,
 *    plane 1 = h).  Weights and biases are "[G][D]" (gate-major).
 *  - Every call validates its arguments before launching anything and
 *    returns a status; nothing throws across the ABI.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Outputs are valid once the stream has completed.  Only a
 *    non-NULL report makes pararnn_newton_solve wait for the stream.
 *  - Without a report, a call is only kernel launches on `stream` (no
 *    allocation, no memset node, no synchronisation), so it can be captured
 *    in a HIP graph.  Each call clears its workspace with a kernel first, so
 *    graph replays do not see each other's look-back words.
 *  - `ws` is a device workspace of at least the queried size, 256-byte
 *    aligned, whose contents need not be initialised.  Calls that overlap in
 *    time must use distinct workspaces.
 *  - Arithmetic is fp32 throughout; bf16 is a storage format for the gate
 *    pre-activations only.
 */
#ifndef PARARNN_H
#define PARARNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARARNN_ABI_VERSION 6
/* upper bound of Newton iterations per call (report.residual holds one more) */
#define PARARNN_MAX_ITERS 64
/* most Newton iterations one fused launch runs (pararnn_newton_opts.fuse_iters) */
#define PARARNN_MAX_FUSE 8

typedef enum {
  PARARNN_OK = 0,
  PARARNN_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad enum, K outside [1, 64], misalignment */
  PARARNN_ERR_UNSUPPORTED = -2,  /* valid but not built: D not a multiple of 2, or too large a grid */
  PARARNN_ERR_WORKSPACE = -3,    /* ws NULL/misaligned or ws_bytes below the queried size */
  PARARNN_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  PARARNN_ERR_DIVERGED = -5      /* tolerance mode: a non-finite max residual, or the budget spent without
                                    convergence and the last residual above the starting one (see tol);
                                    the report is still filled */
} pararnn_status;

typedef enum { PARARNN_F32 = 0, PARARNN_BF16 = 1 } pararnn_dtype;

/* Cells.  G = gate planes, S = state size.
 *  LINEAR    G=2 (a, b), S=1:  h' = a_t h + b_t  (the pre-activation planes ARE the coefficients)
 *  DIAG_GRU  G=3 (z, r, c), S=1, diagonal recurrent weights (a_z, a_r, a_c), biases (b_z, b_r, b_c):
 *              z = sig(U_z + a_z h + b_z),  r = sig(U_r + a_r h + b_r),
 *              c = tanh(U_c + a_c (r h) + b_c),  h' = (1 - z) h + z c
 *  DIAG_LSTM G=4 (i, f, o, g), S=2 with state (c, h), diagonal recurrent weights acting on h:
 *              i, f, o = sig(U + w h + b),  g = tanh(U_g + w_g h + b_g),
 *              c' = f c + i g,  h' = o tanh(c')
 *  DIAG_SLSTM G=4 (z, i, f, o), S=4 with state (c, n, m, h): the sLSTM that the pararnn-torch
 *             README names (ParaSLSTM, mix="diag"; "API overview", "Method") in its published
 *             form, exponential input gate, sigmoid forget gate and log-domain stabiliser m,
 *             diagonal recurrent weights acting on h:
 *              u_g = U_g + w_g h + b_g,  z = tanh(u_z),  o = sig(u_o),  lf = log sig(u_f),
 *              m' = max(lf + m, u_i),  i' = exp(u_i - m'),  f' = exp(lf + m - m'),
 *              c' = f' c + i' z,  n' = f' n + i',  h' = o c' / n'
 *             (at a tie of the max the forget branch is taken).  Its Newton iteration wants a few
 *             Picard sweeps first (opts.picard_iters); it has no measured budget (max_iters > 0).
 *  HEAD_GRU  G=3 (z, r, c), S=1: the head-wise block GRU of the pararnn-torch README ("Usage":
 *             ParaGRU in its head-wise mixing mode: block-diagonal recurrent matrices, factorized Newton).  The D
 *             channels form D / head_size heads of head_size consecutive channels; each gate's
 *             recurrent matrix is block-diagonal with one dense head_size x head_size block per head:
 *              z = sig(U_z + A_z h + b_z),  r = sig(U_r + A_r h + b_r),
 *              c = tanh(U_c + A_c (r h) + b_c),  h' = (1 - z) h + z c
 *             w is [3][D / head_size][head_size][head_size] (block row = output channel, column =
 *             input channel), bias [3][D].  Newton uses the exact block Jacobian; the linear system
 *             splits into one block-bidiagonal system per (batch row, head).  head_size 16, 32 or 64
 *             (others UNSUPPORTED); no measured budget (max_iters > 0). */
typedef enum { PARARNN_CELL_LINEAR = 0, PARARNN_CELL_DIAG_GRU = 1, PARARNN_CELL_DIAG_LSTM = 2,
               PARARNN_CELL_DIAG_SLSTM = 3, PARARNN_CELL_HEAD_GRU = 4 } pararnn_cell;

typedef struct {
  int32_t cell;          /* pararnn_cell */
  int32_t pre_dtype;     /* pararnn_dtype of pre[] */
  int64_t B, T, D;       /* batch, time steps, channels; each >= 0 (an empty problem is a no-op);
                            D must be even                                                     */
  const void* pre[4];    /* G gate pre-activation planes [B][T][D], caller-precomputed
                            (x_t already projected); 8-byte aligned                            */
  const float* w;        /* [G][D] diagonal recurrent weights (ignored for LINEAR); HEAD_GRU:
                            [3][D/head_size][head_size][head_size] dense blocks                   */
  const float* bias;     /* [G][D] biases (ignored for LINEAR)                                 */
  const float* s0;       /* [S][B][D] initial state h_{-1}; NULL = zeros                        */
  const int32_t* cu_seqlens; /* packed sequences, or NULL for one sequence per batch row: n_seqs+1
                                nondecreasing offsets into T (device memory); sequence j covers steps
                                cu_seqlens[j] .. cu_seqlens[j+1]-1 of every batch row.  The state
                                entering each sequence after the first is zero (s0 is the first one's
                                initial state) and nothing flows across a boundary, forward or in the
                                VJP.  Only the offsets strictly between 0 and T matter; the library
                                does not read them on the host, so it cannot check their order.    */
  int64_t n_seqs;        /* number of packed sequences (ignored when cu_seqlens is NULL)          */
  int64_t head_size;     /* HEAD_GRU: channels per head (divides D); ignored by the other cells     */
} pararnn_problem;

/* First Newton iterate when no init_guess is given.  WARM is the GRU / LSTM warm start of the
 * pararnn-torch README ("Method"): every step's state is the cell applied to a zero previous state,
 * H^0_t = f(0, x_t) (for every t, s0 included: the guess does not use s0).  It is computed inside
 * iteration 0's kernel from the gate inputs it loads anyway (no extra pass, no extra buffer).      */
typedef enum { PARARNN_INIT_ZERO = 0, PARARNN_INIT_WARM = 1 } pararnn_init_mode;

typedef struct {
  int32_t max_iters;       /* Newton budget K, 1..PARARNN_MAX_ITERS, or 0 = automatic: the measured
                              K*(T) of pararnn_newton_budget for this cell, init_mode and T         */
  float tol;               /* <= 0: run exactly max_iters iterations.
                              > 0: iteration k evaluates R_k = max|r(H^k)| over b, t, d and state
                              components; the first iteration with R_k < tol is the last one (its
                              update is applied).  A non-finite R_k stops the solve (DIVERGED).  A
                              solve that spends its budget without convergence and whose last R
                              exceeds R_{k0}, the residual at the first Newton (not Picard) iteration
                              k0 = picard_iters, has diverged too (DIVERGED; pararnn-torch README,
                              "Evaluation": a divergence error with the residual history).  A rise
                              from one iteration to the next alone is not divergence: on this
                              triangular system Newton is exact after T updates, and converging LSTM
                              and sLSTM solves show a few rising iterations first.                 */
  const float* init_guess; /* [S][B][T][D] first iterate H^0, or NULL (then init_mode decides).  May
                              equal s_out (resume from a previous solve's output).                  */
  int32_t final_residual;  /* nonzero: one extra pass computes max|r| of the returned trajectory   */
  int32_t init_mode;       /* pararnn_init_mode; ignored when init_guess is non-NULL                 */
  int32_t picard_iters;    /* the first min(picard_iters, K) of the K updates are Picard sweeps
                              H^{k+1}_t = f(H^k_{t-1}, x_t) (the scan element's A set to 0) instead
                              of Newton updates (pararnn-torch README, "API overview": Picard
                              iterations warm the first guess); 0..PARARNN_MAX_ITERS             */
  int32_t fuse_iters;      /* iterations per launch of pararnn_newton_solve (diagonal GRU and LSTM;
                              the other cells, and solves with Picard sweeps, always use one launch
                              per iteration).  1: one launch per iteration.  m in 2..PARARNN_MAX_FUSE:
                              up to m iterations in one launch that reads the gate inputs and the
                              first iterate once and keeps the trajectory in registers between them.
                              0: the library's choice (fixed budget: PARARNN_MAX_FUSE; tolerance
                              mode with tol <= 1e-4: the iteration count tolerance mode reached in
                              the K*(T) campaign of pararnn_newton_budget, same cell, first iterate
                              and length, at the nearest of 1e-4, 1e-5, 1e-6 at or above tol;
                              looser tol: K*(T)).  The result, the report and
                              the residuals are the same, bit for bit, for every value.  In
                              tolerance mode the first launch runs its m iterations without waiting
                              for the stop rule; when the rule met an earlier one, a second launch
                              recomputes the trajectory from the first iterate with the right count
                              (so a solve whose init_guess overlaps s_out uses one launch per
                              iteration there), and single launches follow for the iterations past
                              m.  That second launch and the single launches after the first mostly
                              find the stop rule met: they run on as many workgroups as the device
                              holds at once, looping over the tiles, so exiting costs a few
                              microseconds.  Workspace: one set of look-back words per fused
                              iteration.                                                          */
} pararnn_newton_opts;

typedef struct {          /* (host) */
  int32_t iters;          /* Newton updates applied (kernels that did work)                          */
  int32_t converged;      /* tolerance mode: 1 if some R_k < tol; fixed mode: 0                      */
  int32_t n_residual;     /* entries of residual[] that are set                                      */
  float residual[PARARNN_MAX_ITERS + 1]; /* R_0 .. R_{iters-1}; then, if final_residual was asked,
                                            the max residual of the returned trajectory            */
} pararnn_report;

/* ------------------------------------------------------------------------------------------------
 * pararnn_newton_solve -- Newton solve of F(H) = 0 for the given cell (pararnn-torch README,
 * "Method"; ParaRNN abstract).  For the diagonal cells each iteration is ONE fused kernel: it
 * evaluates the residual and the per-channel Jacobian (scalar for GRU, 2x2 for LSTM, 4x4 for sLSTM)
 * at the current iterate, forms the affine scan elements of the linearised recurrence in registers,
 * combines them across the workgroup and across time chunks (decoupled look-back), and writes
 * H^{k+1} = H^k + delta in place into s_out.  For HEAD_GRU an iteration is three kernels: each
 * chunk's composed map of dense Jacobian blocks (MFMA), a carry of the state across chunks, and a
 * per-step replay that writes H^{k+1} in place.
 *   s_out  [S][B][T][D] fp32 output trajectory (H^{iters}).  Must not overlap pre/w/bias/s0.
 *   report (host, nullable): when given, the call waits for the stream and fills it.
 * Several iterations can share one launch (opts.fuse_iters): the same per-iteration arithmetic, with
 * the gate inputs read once and the trajectory kept in registers between iterations.
 * Errors: INVALID_ARG / UNSUPPORTED / WORKSPACE before any launch; HIP after a failed launch;
 * DIVERGED (tolerance mode, report given) when a max residual is NaN or Inf, or when the budget ran out
 * above the starting residual (see tol).  Without a report the call only launches and returns OK; the
 * status is then available, after the stream has completed, from pararnn_newton_report on the same
 * workspace (with final_residual = 0 it launches nothing and reads the residual history the solve left).
 * The workspace size depends on opts (fused iterations); opts = NULL gives a size that fits every
 * option.  Contents need not be preserved between solves.
 * ---------------------------------------------------------------------------------------------- */
size_t pararnn_newton_workspace_bytes(const pararnn_problem* prob, const pararnn_newton_opts* opts);
pararnn_status pararnn_newton_solve(const pararnn_problem* prob, const pararnn_newton_opts* opts,
                                    float* s_out, void* ws, size_t ws_bytes, void* stream,
                                    pararnn_report* report);

/* pararnn_newton_solve_noalloc -- pararnn_newton_solve without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is a static device array of PARARNN_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends; the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).  The first call on each device looks up that device's address of the
 * array (hipGetSymbolAddress, with the device current): make it outside graph capture.
 *   Same arguments, results, report and errors as pararnn_newton_solve, bit for bit.  With
 * opts->fuse_iters = 0 the launch length is the library's, shortened until the look-back words fit the
 * array; a problem whose workspace does not fit even at one launch per iteration (or at an explicit
 * fuse_iters) returns PARARNN_ERR_WORKSPACE before launching anything.
 *   All calls on one GPU share its array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be made.  Each call clears the parts that must start at zero with a kernel,
 * so the previous call's contents do not matter. */
#define PARARNN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
pararnn_status pararnn_newton_solve_noalloc(const pararnn_problem* prob, const pararnn_newton_opts* opts,
                                            float* s_out, void* stream, pararnn_report* report);

/* The same solve in three steps, for callers that time, checkpoint or interleave work between
 * iterations.  pararnn_newton_solve(...) with fuse_iters = 1 is exactly: prepare; iterate k = 0 ..
 * max_iters-1; [final residual]; report (with fused launches it returns the same bits).  All share
 * one workspace and stream; `opts` must be the same object contents in every call of one solve.
 *   prepare  -- clears the workspace's counters and look-back words (one small kernel).
 *   iterate  -- launches iteration k (0 <= k < max_iters): the kernels of one iteration, reading H^k
 *               (init_guess for k = 0, else s_out) and writing H^{k+1} into s_out.  In tolerance mode a kernel
 *               whose earlier residual met the stop rule exits at once without touching s_out.
 *   report   -- (host) optionally launches the final-residual pass, waits for the stream and fills
 *               `report`; returns DIVERGED as pararnn_newton_solve does.                              */
pararnn_status pararnn_newton_prepare(const pararnn_problem* prob, const pararnn_newton_opts* opts,
                                      void* ws, size_t ws_bytes, void* stream);
pararnn_status pararnn_newton_iterate(const pararnn_problem* prob, const pararnn_newton_opts* opts,
                                      int k, float* s_out, void* ws, size_t ws_bytes, void* stream);
pararnn_status pararnn_newton_report(const pararnn_problem* prob, const pararnn_newton_opts* opts,
                                     const float* s_out, void* ws, size_t ws_bytes, void* stream,
                                     pararnn_report* report);

/* ------------------------------------------------------------------------------------------------
 * pararnn_linear_scan -- the linear recurrence every Newton step reduces to (pararnn-torch README,
 * "Method": the linearised system is solved by a parallel scan along time), as a single-pass scan.
 *   forward (reverse = 0): s_{-1} = s0,  s_t = A_t s_{t-1} + b_t,  t = 0 .. T-1
 *   reverse (reverse = 1): s_T    = s0,  s_t = A_t s_{t+1} + b_t,  t = T-1 .. 0
 *   S = 1: a [B][T][D], b [B][T][D];  S = 2: a [4][B][T][D] (A00, A01, A10, A11), b [2][B][T][D].
 *   dtype: storage of a and b (fp32 or bf16).  s0 [S][B][D] fp32 or NULL (zeros).
 *   cu_seqlens, n_seqs: packed sequences as in pararnn_problem, or NULL: the state entering each
 *         sequence is zero, except s0 for the sequence at the scan's starting end (the first one
 *         forward, the last one in reverse).
 *   s_out [S][B][T][D] fp32; it may alias a or b exactly (fp32 storage), not partially.
 * ---------------------------------------------------------------------------------------------- */
size_t pararnn_scan_workspace_bytes(int S, int64_t B, int64_t T, int64_t D);
pararnn_status pararnn_linear_scan(int S, int64_t B, int64_t T, int64_t D, int dtype,
                                   const void* a, const void* b, const float* s0,
                                   const int32_t* cu_seqlens, int64_t n_seqs, float* s_out,
                                   int reverse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * pararnn_scan_vjp -- gradients at a solved trajectory by the adjoint (pararnn-torch README,
 * "Method": backward follows the paper's adjoint equation).  With dL/dh_t = g_t on the h component:
 *   lambda_{T-1} = e_h g_{T-1},  lambda_t = e_h g_t + J_{t+1}^T lambda_{t+1}   (one reverse scan)
 *   dL/dU_{gate,t} = lambda_t . d f / d u_gate (s_{t-1}, x_t)
 *   dL/dw_gate = sum_{b,t} dL/dU_{gate,t} * (factor of w_gate in u_gate),  dL/dbias = sum dL/dU
 *   dL/ds0 = J_0^T lambda_0
 * LINEAR: d_pre = (dL/da_t = lambda_t h_{t-1}, dL/db_t = lambda_t).  Parameter sums are reduced in a
 * fixed order (bitwise reproducible run to run).
 *   s          [S][B][T][D] fp32 the trajectory the gradient is taken at (normally a solve's output)
 *   g          [B][T][D] fp32 upstream gradient on h
 *   d_pre      [G][B][T][D] fp32 (required)
 *   d_w, d_bias [G][D] fp32 or NULL (ignored for LINEAR)
 *   d_s0       [S][B][D] fp32 or NULL;  lambda_out [S][B][T][D] fp32 or NULL
 * ---------------------------------------------------------------------------------------------- */
size_t pararnn_vjp_workspace_bytes(const pararnn_problem* prob);
pararnn_status pararnn_scan_vjp(const pararnn_problem* prob, const float* s, const float* g,
                                float* d_pre, float* d_w, float* d_bias, float* d_s0,
                                float* lambda_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * pararnn_newton_budget -- (host only, no GPU call) the Newton budget a solve runs: max_iters when
 * it is positive, else K*(T), the smallest K whose iterate agreed with the sequential unroll to 1e-4
 * (max abs) in a measurement on a grid of lengths T (pararnn-torch README, "Method": K*(T) and
 * the automatic iteration count; "Benchmarks": the tau = 1e-4, B = 1 campaign).  The
 * table was measured with the fp64 reference on seeded synthetic inputs (B = 1, D = 1024; gate
 * inputs ~ N(0, 1), recurrent weights ~ U(-0.5, 0.5), biases ~ N(0, 0.01)); a length between grid
 * points takes the next larger point's budget, a length beyond the grid one more than the last.
 * LINEAR always needs 1.  It is a default for inputs like those, not a guarantee: tolerance mode
 * (opts.tol > 0) is the guarantee.  A solve with an init_guess and max_iters = 0 uses the zero-start
 * budget.  Returns K >= 1, or PARARNN_ERR_INVALID_ARG for a bad cell, init_mode, T or max_iters.
 * ---------------------------------------------------------------------------------------------- */
int pararnn_newton_budget(int cell, int init_mode, int64_t T, int max_iters);

/* human-readable text of a status (static storage) */
const char* pararnn_status_string(int status);
/* PARARNN_ABI_VERSION of the built library */
int pararnn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PARARNN_H */
