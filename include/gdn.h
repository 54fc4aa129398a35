/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated DeltaNet prompt-path library (libgdn.so).
 *
 * What the library computes, per value head h, for tokens t = 0 .. T-1, with a
 * dk x dv FP32 state S (row i = key dim, column j = value dim):
 *
 *     S_t = e^{g_t} S_{t-1} + k_t ( beta_t ( v_t - e^{g_t} S_{t-1}^T k_t ) )^T
 *     o_t = S_t^T q_t
 *
 * ("#413 prefill: DeltaNet recurrence with the three value heads of a key head in one
 * thread", sections "What changes" and "Exactness": the kv sum, the delta, the state
 * update and the output sum, evaluated one token at a time.)  Value head h reads key head
 * h mod n_k_heads (same page, "What changes": the heads sharing a key head are h, h+16,
 * h+32 for 16 key heads).  g is the log-decay (g <= 0; the decay factor is e^g).
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a DEVICE pointer owned by the caller (the library never
 *    allocates, frees or keeps a pointer across calls) and must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Each call
 *    validates its arguments on the host, enqueues its kernels on `stream` and returns
 *    without synchronising; results are ready after the caller synchronises the stream.
 *    Kernel faults surface at that synchronisation, as for any HIP library.
 *  - Arguments are validated before anything is enqueued: a rejected call returns a
 *    non-zero gdn_status and changes no memory.  No C++ exception crosses the ABI and
 *    the library prints nothing.
 *  - Only dk = dv = 128 is supported; n_v_heads must be a positive multiple of
 *    n_k_heads with at most 4 value heads per key head; T * n_v_heads * dv must be
 *    below 2^31 (32-bit element offsets) and, for the recurrence and layer calls,
 *    2048 * n_v_heads * dv * 4 below 2^31 (32-bit byte counts over one 2048-token
 *    super-block: n_v_heads <= 2047).
 *    Anything else is GDN_ERR_BAD_SHAPE -- there is no fallback path.
 *  - Layouts (row-major, contiguous, float32 unless stated):
 *        q, k         [T][n_k_heads][dk]   (the library applies no normalisation/scale)
 *        v, o         [T][n_v_heads][dv]
 *        g, beta      [T][n_v_heads]
 *        state_in/out [n_v_heads][dk][dv]
 *        z            [T][n_v_heads][dv]   w [n_v_heads][dv]   y [T][n_v_heads][dv] fp16
 *  - Calls on different streams must not share output buffers or a workspace.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_POINTER = 1, /* a required pointer is NULL                                  */
  GDN_ERR_BAD_SHAPE = 2,    /* T < 0, dk/dv != 128, heads < 1, n_v_heads % n_k_heads != 0,
                               n_v_heads / n_k_heads > 4, T * n_v_heads * dv >= 2^31,
                               n_v_heads > 2047, or a negative / non-finite eps             */
  GDN_ERR_MISALIGNED = 3,   /* a pointer is not 16-byte aligned                            */
  GDN_ERR_ALIASING = 4,     /* an output overlaps an input or another output
                               (state_out == state_in exactly is allowed)                  */
  GDN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than gdn_chunked_workspace_bytes() */
  GDN_ERR_HIP = 6           /* a HIP runtime call or a launch failed: gdn_last_hip_error()  */
};

/*
 * Sequential recurrence: walks the tokens one at a time ("#413 ...", sections "What
 * changes" and "Exactness"; the order within a token is kv sum, delta, update, output).
 *
 *   q, k, v, g, beta : inputs (layouts above), read only.
 *   state_in         : S_0 per value head, read only (may equal state_out).
 *   state_out        : S_T per value head, written.  state_out == state_in is allowed
 *                      (in-place); any other overlap with an input is GDN_ERR_ALIASING.
 *   o                : o_t per token and value head, written.
 *   T = 0            : nothing is written to o; state_in is copied to state_out if they
 *                      differ; returns GDN_OK (o may then be NULL).
 */
int gdn_recurrence_seq(const float* q, const float* k, const float* v, const float* g,
                       const float* beta, const float* state_in, float* state_out, float* o,
                       int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* stream);

/*
 * Bytes of caller-owned device scratch that gdn_recurrence_chunked needs.  It does not
 * depend on T: the scratch holds the per-chunk operators of two 2048-token super-blocks,
 * the one being scanned and the next one being prepared ("#1372 DeltaNet recurrence:
 * STRATA_GDN_CHUNKED=1", section "What it does", paragraph "Scratch": the prep output of
 * a super-block, allocated once per device and kept).  Returns 0 for an unsupported shape.
 */
size_t gdn_chunked_workspace_bytes(int n_k_heads, int n_v_heads, int dk, int dv);

/*
 * Chunked recurrence in the WY form ("#1372 ...", section "What it does"): the same
 * function as gdn_recurrence_seq, computed in chunks of 32 tokens.  Per chunk and value
 * head, with gamma the inclusive running sum of g inside the chunk and S0 the state
 * before it:
 *     A[t][i] = beta_t e^{gamma_t - gamma_i} k_t.k_i   (i < t),   T = (I + A)^-1,
 *     D = T beta (V - e^{gamma} K S0),
 *     O = e^{gamma} Q S0 + P D,  P[t][i] = e^{gamma_t - gamma_i} q_t.k_i  (i <= t),
 *     S' = e^{gamma_last} S0 + K^T e^{gamma_last - gamma} D.
 * A prep kernel forms the chunk operators for every chunk of a 2048-token super-block at
 * once; a scan kernel then walks the super-block's chunks carrying the state on chip.
 * The scan launch of super-block n also carries the prep of super-block n+1 on the
 * compute units the scan leaves idle.  The state passes between super-blocks through
 * state_out.  A last partial chunk is
 * padded with zero tokens (g = 0, beta = 0), which leave the state unchanged.
 *
 *   workspace, workspace_bytes : device scratch of at least
 *                      gdn_chunked_workspace_bytes(...) bytes, 16-byte aligned.  Its
 *                      contents on entry do not matter and on return are unspecified.
 *                      It must not overlap any input or output.  The call uses it until
 *                      its work on `stream` has finished: calls that may run at the same
 *                      time (on different streams) need workspaces of their own.
 *   Other arguments, aliasing rules and T = 0 behave as for gdn_recurrence_seq.
 *   Results differ from gdn_recurrence_seq only by float32 summation order.
 */
int gdn_recurrence_chunked(const float* q, const float* k, const float* v, const float* g,
                           const float* beta, const float* state_in, float* state_out,
                           float* o, int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Profiling variant of gdn_recurrence_chunked: the same validation and the same work on
 * the same stream; in addition it records the caller's events scan_events[2i] and
 * scan_events[2i+1] (hipEvent_t values, created by the caller) on `stream` immediately
 * before and after the scan kernel of super-block i, for every i with 2i+1 <
 * n_scan_events.  This lets a caller time the scan kernel alone without a profiler.
 * scan_events may be NULL only when n_scan_events <= 0 (then this is
 * gdn_recurrence_chunked exactly).
 */
int gdn_recurrence_chunked_timed(const float* q, const float* k, const float* v,
                                 const float* g, const float* beta, const float* state_in,
                                 float* state_out, float* o, int64_t T, int n_k_heads,
                                 int n_v_heads, int dk, int dv, void* workspace,
                                 size_t workspace_bytes, void* const* scan_events,
                                 int n_scan_events, void* stream);

/*
 * Gated RMS output norm to FP16 ("#413 ...", section "What changes": the output norm
 * reads the FP32 recurrence output and writes only the FP16 copy y_h that the out
 * projection reads; the pages print no formula, and the library takes the plain reading
 * of a gated RMS norm with a per-value-head weight and a sigmoid gate):
 *
 *   y[t][h][j] = fp16_rne( o[t][h][j] * rsqrt(mean_j o[t][h][:]^2 + eps)
 *                          * w[h][j] * sigmoid(z[t][h][j]) )
 *
 *   o, z, w : inputs (layouts above), read only.  eps >= 0 (a negative or non-finite eps
 *             is GDN_ERR_BAD_SHAPE).  The mean of squares is accumulated in FP32, so a row
 *             whose largest |o| exceeds about 1.6e18 overflows it (its y is then 0); an
 *             all-zero row with eps = 0 gives NaN, as the formula does.
 *   y       : output, IEEE binary16 bit patterns, rounded to nearest even.  Must not
 *             overlap o, z or w.
 *   T = 0   : nothing is written; returns GDN_OK.
 */
int gdn_out_norm(const float* o, const float* z, const float* w, float eps, uint16_t* y,
                 int64_t T, int n_v_heads, int dv, void* stream);

/*
 * The recurrence with the kernel chosen by T: gdn_recurrence_seq for T < GDN_CHUNKED_MIN_T,
 * gdn_recurrence_chunked otherwise (same arguments and results as the call it picks).
 * ("#1372 DeltaNet recurrence: STRATA_GDN_CHUNKED=1", sections "What it does" and
 * "Measured": the chunked path loses to the sequential kernel for short prompts, and the
 * pages set a minimum length for it on their card.  On an MI355X the two cross between 48
 * and 64 tokens: 16 tokens take 29 vs 37 us, 32 tokens 33 vs 37 us, 48 tokens 36 vs 39
 * us, 64 tokens 40 vs 39 us, 128 tokens 55 vs 44 us, host clock around one call and its
 * synchronisation.)  The workspace may be NULL when T < GDN_CHUNKED_MIN_T.
 */
#define GDN_CHUNKED_MIN_T 56
int gdn_recurrence(const float* q, const float* k, const float* v, const float* g,
                   const float* beta, const float* state_in, float* state_out, float* o,
                   int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * One layer's prompt path: the chunked recurrence (gdn_recurrence_chunked, same
 * arguments, same results bit for bit) followed by the gated RMS output norm
 * (gdn_out_norm with z, w, eps, y, same results bit for bit), in one call.  The norm of
 * each 2048-token super-block runs inside the recurrence launch of the next super-block,
 * on waves the scan leaves free, so it costs next to nothing; only the last super-block's
 * norm is a launch of its own.  The FP32 output o is still written (it is the norm's
 * input and a result of the call).
 *
 * ("#1372 DeltaNet recurrence: STRATA_GDN_CHUNKED=1", section "What it does", for the
 * recurrence; "#413 ...", section "What changes", for the norm, which the pages keep as a
 * separate kernel after the recurrence: running it inside the next recurrence launch is
 * this library's arrangement.)
 *
 *   z, w, eps, y : as for gdn_out_norm.  y must not overlap any other argument; o, the
 *                  state and the workspace must not overlap z or w.
 *   Everything else as for gdn_recurrence_chunked.  T = 0 copies the state and writes
 *   nothing else.
 */
int gdn_layer_chunked(const float* q, const float* k, const float* v, const float* g,
                      const float* beta, const float* state_in, float* state_out, float* o,
                      const float* z, const float* w, float eps, uint16_t* y, int64_t T,
                      int n_k_heads, int n_v_heads, int dk, int dv, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * gdn_layer_chunked that additionally records caller-created hipEvent_t handles around
 * each recurrence launch (the launch of super-block sb between scan_events[2 sb] and
 * scan_events[2 sb + 1], for 2 sb + 1 < n_scan_events), on `stream`.  For timing.
 */
int gdn_layer_chunked_timed(const float* q, const float* k, const float* v, const float* g,
                            const float* beta, const float* state_in, float* state_out,
                            float* o, const float* z, const float* w, float eps, uint16_t* y,
                            int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                            void* workspace, size_t workspace_bytes,
                            void* const* scan_events, int n_scan_events, void* stream);

/*
 * The step before the recurrence ("Round 20 Track C Audit: gdn_pre ...", section 1: the
 * 4-tap causal conv of the projection output and the key-head branch that normalises q and
 * k; section 2 lists its outputs, the normalised q and k, the convolved v, the gate and
 * beta, and the conv history).  Per token t and channel c of x:
 *
 *   u[t][c]   = sum_{j=0..3} conv_w[c][j] * xe[t + j][c]
 *               (xe = the 3 rows of hist_in, oldest first, followed by the T rows of x:
 *               tap 3 multiplies the current token)
 *   u         = act(u)            activation 0: none; 1: SiLU, u / (1 + e^-u)
 *   q[t][kh]  = u_q / sqrt(sum u_q^2 + eps) / sqrt(dk)      (per key head, over dk)
 *   k[t][kh]  = u_k / sqrt(sum u_k^2 + eps)
 *   v[t][h]   = u_v
 *   g[t][h]   = -exp(A_log[h]) * log(1 + exp(a[t][h] + dt_bias[h]))
 *   beta[t][h]= 1 / (1 + exp(-b[t][h]))
 *   hist_out  = the last 3 rows of xe (the history of the next call of the same sequence)
 *
 * The page shows the conv, the history and the normalised outputs but prints neither the
 * activation, nor the form of eps, nor the gate and beta formulas: those are this
 * library's readings (the activation is an argument).
 *
 *   x          [T][C] fp32, C = (2 n_k_heads + n_v_heads) * 128: the q channels of key head
 *              kh at kh*128, the k channels of key head kh at (n_k_heads + kh)*128, the v
 *              channels of value head h at (2 n_k_heads + h)*128.
 *   conv_w     [C][4], hist_in [3][C]: read.  hist_out [3][C]: written; it must not overlap
 *              hist_in (pass a second buffer and swap them between calls).
 *   a, b       [T][n_v_heads], A_log, dt_bias [n_v_heads]: read.  g, beta [T][n_v_heads]:
 *              written.  These six are all given or all NULL (then no gate and beta).
 *   q, k       [T][n_k_heads][dk], v [T][n_v_heads][dv]: written (the recurrence's layout).
 *   eps        >= 0 and finite; activation 0 or 1; dk = dv = 128.  Otherwise, or when the
 *              grid would reach 2^31 waves or workgroups (one wave per 32 tokens of each
 *              128-channel head block, one thread per gate value), GDN_ERR_BAD_SHAPE.
 *   T = 0      copies hist_in to hist_out and writes nothing else (every pointer but the
 *              two histories may then be NULL).
 *   No output may overlap an input or another output.  The results are FP32: within a few
 *   FP32 ulps of the exact values (the conv, exp and log are the correctly rounded or
 *   1-ulp library functions).
 */
int gdn_pre(const float* x, const float* conv_w, const float* hist_in, float* hist_out,
            const float* a, const float* b, const float* A_log, const float* dt_bias,
            int activation, float eps, float* q, float* k, float* v, float* g, float* beta,
            int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* stream);

/*
 * gdn_layer_chunked for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same validation, the
 * same kernels and the same results bit for bit as gdn_layer_chunked, but without a
 * workspace argument: the chunked kernels' scratch is a file-scope device array of the
 * library, 68 MiB per device, which each device holds from the first call on it until the
 * process ends.  The call itself allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine); the caller still passes every input and output.
 *
 *   n_v_heads        : at most 64 (the array holds the operators of two 2048-token
 *                      super-blocks of 64 value heads); more is GDN_ERR_WORKSPACE.
 *   first call       : on a device, resolves the array's device address (with that
 *                      device current); make it outside any graph capture.
 *   concurrency      : every call on a device uses that device's one array, which keeps
 *                      the last call's contents (no call depends on them).  Calls on one
 *                      stream are ordered; calls that overlap on one device (different
 *                      streams, or several host threads' streams) race on the array and
 *                      give undefined results.
 *   Everything else  : as for gdn_layer_chunked.
 */
int gdn_layer_chunked_noalloc(const float* q, const float* k, const float* v, const float* g,
                              const float* beta, const float* state_in, float* state_out,
                              float* o, const float* z, const float* w, float eps, uint16_t* y,
                              int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                              void* stream);

/* A static, never-NULL description of a gdn_status value. */
const char* gdn_status_string(int status);

/* The hipError_t of the most recent GDN_ERR_HIP returned on the calling thread
   (0 if none). */
int gdn_last_hip_error(void);

/* Version of this ABI (incremented on any incompatible change). */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
