/*
 * dspark.h -- C ABI of the DSpark draft -> schedule -> verify hot path, gfx950.
 *
 * Three calls, following the problem statement on the pages that describe
 * DSpark ("DSpark: Confidence-Scheduled Speculative Decoding with
 * Semi-Autoregressive Generation", sections 2.1, 3.1, 3.2.2; restated in
 * "Speculative decoding, from zero to DSpark", sections 2, 6, 8):
 *
 *   dspark_markov_draft  the sequential Markov head: adds W1[x_{k-1}] W2 to
 *                        the backbone's base logits U_k, softmax, samples x_k
 *                        left to right and keeps exact draft probabilities;
 *   dspark_schedule      Algorithm 1: prefix-survival products, global sort,
 *                        greedy admission against the SPS(B) cost table;
 *   dspark_verify        rejection sampling over the flattened
 *                        variable-length verify batch: accept with
 *                        min(1, p/q), resample the first rejection from
 *                        norm(max(0, p - q)), else draw a bonus token from p.
 *
 * Conventions (all calls):
 *   - Array arguments are DEVICE pointers to caller-owned, contiguous,
 *     row-major buffers.  The library never allocates, frees or retains them
 *     and performs no host<->device synchronisation.  Scratch memory is the
 *     caller-supplied `workspace` (size from the matching *_workspace_bytes
 *     query, 256-byte aligned).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - The return value is a status.  Shape, pointer, dtype and workspace
 *     errors are detected on the host before anything is enqueued (nothing is
 *     written).  DSPARK_E_HIP means a launch failed.  Data-dependent errors
 *     (token ids out of range, inconsistent cu_seqlens, confidences outside
 *     [0, 1]) are reported through the outputs as documented per call; kernels
 *     never read or write outside the buffers described here.
 *   - Randomness: every random decision consumes one uniform
 *     u = (w >> 8) * 2^-24 where w is the first word of Philox4x32-10
 *     (Salmon et al., SC'11) with key (seed lo, seed hi) and counter
 *     (step lo, step hi, request index, (position << 2) | purpose),
 *     purpose 0 = draft sample, 1 = accept test, 2 = correction/bonus sample.
 *     Every categorical draw is an inverse-CDF draw in ascending token id.
 *   - Temperature T > 0 divides both draft and target logits; T == 0 selects
 *     greedy decoding (first argmax; verify accepts iff argmax p == x).
 *   - The Markov factors are bf16.  W1 is the V x r embedding table (row v at
 *     W1 + v*r).  W2 (r x V in the pages' notation) is passed column-major:
 *     column v, the r weights that produce logit v, is contiguous at W2 + v*r.
 *     r must be a multiple of 8 and at most DSPARK_MAX_RANK; r == 0 means no
 *     Markov head (W1 and W2 may then be NULL).
 *   - Each logit buffer (U, P, D) and each Markov factor must be smaller than
 *     4 GiB (kernels address them with 32-bit byte offsets); larger inputs
 *     return DSPARK_E_SHAPE.
 *   - Empty batches: a call with no requests (B or R == 0; n == 0 for
 *     dspark_uniforms) and otherwise valid sizes and scalars returns DSPARK_OK
 *     without enqueuing anything; its array and workspace pointers are not
 *     read and may be NULL.  dspark_schedule and dspark_schedule_async are the
 *     exception: with R == 0 they still write the empty layout (see there).
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dspark_status {
  DSPARK_OK = 0,
  DSPARK_E_NULL = -1,      /* a required pointer is NULL */
  DSPARK_E_SHAPE = -2,     /* a dimension is out of its documented range */
  DSPARK_E_DTYPE = -3,     /* dtype code not supported for that argument */
  DSPARK_E_RANGE = -4,     /* a scalar argument is out of range (temperature, mode, table length) */
  DSPARK_E_WORKSPACE = -5, /* workspace NULL or smaller than the query */
  DSPARK_E_HIP = -6        /* a HIP launch failed */
};

enum dspark_dtype { DSPARK_F32 = 0, DSPARK_BF16 = 1 };

enum dspark_sched_mode {
  DSPARK_SCHED_EARLY_STOP = 0, /* Algorithm 1: break at the first Theta <= Theta_best */
  DSPARK_SCHED_GLOBAL = 1,     /* no break: best Theta on the sorted path (earliest on ties) */
  DSPARK_SCHED_TOPK = 2        /* admit the first min(capacity, |E|) candidates */
};

#define DSPARK_MAX_K 16              /* draft positions per request */
#define DSPARK_MAX_RANK 256          /* Markov rank r */
#define DSPARK_MAX_CANDIDATES 16384  /* R * K for dspark_schedule */
#define DSPARK_STS_MAX_BINS 32        /* ECE bins for dspark_sts_fit */
#define DSPARK_STS_MAX_GRID 65535     /* grid temperatures for dspark_sts_fit */

/* Human-readable text for a status code (static storage). */
const char* dspark_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int dspark_version(void);

/* The 16 hex digits identifying the sources the library was built from
 * (SHA-256 over the source files and compiler flags); static storage. */
const char* dspark_build_id(void);

/* ------------------------------------------------------------------------ *
 * W2 in MFMA fragment order, made once per weight load.  DSpark paper
 * section 3.1 ("Markov head": W2 is the r x V logit projection every
 * position multiplies by).
 *
 * The bias MFMAs read W2 in 1 KB fragments, each the 16-byte pieces of 64
 * lanes in lane order; dspark_markov_prepare_w2 writes that copy of the
 * column-major W2 into caller memory W2f (W2f_bytes >=
 * dspark_markov_w2_frag_bytes(V, r) = ceil(V / 64) * 4 * ceil(r / 32) KB,
 * 16-byte aligned), zeros past V and past r.  The copy depends on W2 only:
 * made once, it serves every dspark_markov_draft, dspark_verify and
 * dspark_acceptance_label call on the same W2 (argument W2f), which then
 * neither rebuild it nor need workspace for it.  The copy must be smaller
 * than 4 GiB.  r == 0: nothing to prepare (0 bytes, no launch).
 * ------------------------------------------------------------------------ */
size_t dspark_markov_w2_frag_bytes(int V, int r);
int dspark_markov_prepare_w2(int V, int r, const void* W2, void* W2f, size_t W2f_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Sequential Markov-head draft.  DSpark paper section 3.1 ("Sequential
 * stage", "Markov head"); "Speculative decoding, from zero to DSpark",
 * section 6 and Appendix A4.
 *
 * For k = 1..K in order and every request b:
 *   z_k = (U[b,k-1,:] + W1[x_{k-1},:] W2) / T,  x_0 = x0[b]   (bias at every k)
 *   x_k = inverse-CDF draw from softmax(z_k) with the uniform of (b, k, draft)
 * Outputs (each [B, K]):
 *   x_out      drafted token ids;
 *   q_tok_out  q_k(x_k), the exact draft probability of the drawn token (1 when T == 0);
 *   lse_out    log sum_v exp(z_k(v)) in natural-log units (when T == 0: the
 *              largest biased logit).
 * Inputs: U [B, K, V] (u_dtype f32 or bf16); W1 [V, r] and W2 (column-major
 * r x V) bf16; W2f the copy of W2 made by dspark_markov_prepare_w2, or NULL
 * (the call then makes it in its workspace, about 27 us at V = 151936,
 * r = 256); x0 [B] int32.  Limits: 0 <= B, 1 <= K <= DSPARK_MAX_K, 1 <= V,
 * r as in the header comment, U smaller than 4 GiB.
 * Data errors: an anchor (or the previous drawn token) outside [0, V) makes
 * that request's remaining positions x = -1, q_tok = lse = NaN.
 * Workspace: 256-byte aligned, contents need not be initialised: the
 * per-slice softmax partials (dspark_markov_draft_workspace_bytes(B, K, V, 0)
 * bytes) and, when r > 0 and W2f is NULL, the fragment-ordered copy of W2
 * after them (dspark_markov_draft_workspace_bytes(B, K, V, r) bytes in all).
 * ------------------------------------------------------------------------ */
size_t dspark_markov_draft_workspace_bytes(int B, int K, int V, int r);
int dspark_markov_draft(int B, int K, int V, int r, float temperature,
                        const void* U, int u_dtype,
                        const void* W1, const void* W2, const void* W2f,
                        const int32_t* x0,
                        uint64_t seed, uint64_t step,
                        int32_t* x_out, float* q_tok_out, float* lse_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Markov draft with the confidence head of every position, in one call.
 * DSpark paper sections 3.1 (Markov head) and 3.2.1 (Confidence Head: the
 * head reads the Markov feature of the previously sampled token);
 * "Speculative decoding, from zero to DSpark", section 8.
 *
 * The outputs of dspark_markov_draft (same arguments, same meaning, bit for
 * bit the same values) and those of dspark_confidence_head on the drafted
 * tokens (x0, x_out), bit for bit the same values as that call:
 *   z[b, k] = w_h . H[b, k] + w_e . W1[x_{b,k-1}] + bias,  x_{b,0} = x0[b]
 *   c_out[b, k] = sigmoid(z[b, k] / T_k)
 * The head runs as one launch after the draft's last position, on the same
 * stream.  Head inputs: d the hidden width; H [B, K, d] (h_dtype);
 * w_h [d] f32; w_e [r] f32 (unused when r == 0); sts_temperature [K] f32 or
 * NULL (T_k = 1).  Head outputs: c_out [B, K] f32; logit_out [B, K] f32 (z)
 * or NULL.  Limits and data errors: those of both calls (a previous token
 * outside [0, V) gives c = z = NaN).  Workspace: as dspark_markov_draft.
 * ------------------------------------------------------------------------ */
int dspark_markov_draft_with_confidence(int B, int K, int V, int r, float temperature,
                                        const void* U, int u_dtype,
                                        const void* W1, const void* W2, const void* W2f,
                                        const int32_t* x0,
                                        uint64_t seed, uint64_t step,
                                        int32_t* x_out, float* q_tok_out, float* lse_out,
                                        int d, const void* H, int h_dtype,
                                        const float* w_h, const float* w_e, float bias,
                                        const float* sts_temperature,
                                        float* c_out, float* logit_out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Hardware-aware prefix scheduler.  DSpark paper section 3.2.2, Algorithm 1
 * (modes GLOBAL and TOPK: section 5.2); "Speculative decoding, from zero to
 * DSpark", section 8.
 *
 *   a[r,j] = c[r,1] * ... * c[r,j]   (float32, one rounding per factor)
 *   candidates (r, j) with a > 0, sorted by a descending, then j ascending,
 *   then r ascending; admitted greedily from B = R, tau = R, Theta = tau*SPS(B).
 *   tau is accumulated in int64 fixed point (each a adds floor(a * 2^32));
 *   Theta = double(tau) * 2^-32 * sps[B].
 * Inputs: c [R, K] f32 in [0, 1]; sps [sps_len] f64, steps/s indexed by the
 * verify batch size B (tokens), sps_len > R * (K + 1); capacity (TOPK only) >= 0.
 * Outputs: a_out [R, K] f32; ell_out [R] int32 (verify lengths l*_r);
 * cu_seqlens_out [R + 1] int32 (prefix sums of 1 + l*_r, the flattened verify
 * layout); n_admitted_out [1] int32; theta_out [1] f64 (Theta of the choice).
 * Limits: 0 <= R, 1 <= K <= DSPARK_MAX_K, R * K <= DSPARK_MAX_CANDIDATES.
 * R == 0 (empty batch: nothing to admit, B = tau = 0): cu_seqlens_out[0] = 0,
 * n_admitted = 0, theta = 0 * sps[0]; c, a_out, ell_out may be NULL and no
 * workspace is needed.
 * Data errors: any c outside [0, 1] or NaN gives ell = 0, cu_seqlens[r] = r,
 * n_admitted = -1, theta = NaN (a valid no-draft layout).
 * Workspace: dspark_schedule_workspace_bytes(R, K) bytes (the sorted
 * candidate keys, each candidate's rank and two counters), caller-owned,
 * contents need not be initialised.
 * Two launches: candidate ranks across many workgroups, then one workgroup
 * for the admission scan and the layout.
 * ------------------------------------------------------------------------ */
size_t dspark_schedule_workspace_bytes(int R, int K);
int dspark_schedule(int R, int K, const float* c,
                    const double* sps, int sps_len,
                    int mode, int capacity,
                    float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out,
                    int32_t* n_admitted_out, double* theta_out,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------------------------------------ *
 * dspark_schedule without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, outputs, limits, data
 * errors and results as dspark_schedule, minus the workspace: the sorted
 * candidate keys, the candidates' ranks and two counters go to a
 * library-owned device array sized for DSPARK_NOALLOC_MAX_CANDIDATES
 * candidates (192.25 KB on each GPU the library runs on, held until the
 * process ends).  The call allocates nothing and
 * calls no allocating routine; R * K above DSPARK_NOALLOC_MAX_CANDIDATES
 * returns DSPARK_E_SHAPE.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race on
 * it and must be ordered by the caller.  Nothing in the array needs to start
 * at zero (each call writes every key, rank and counter it reads).
 * ------------------------------------------------------------------------ */
#define DSPARK_NOALLOC_MAX_CANDIDATES 16384
int dspark_schedule_noalloc(int R, int K, const float* c,
                            const double* sps, int sps_len,
                            int mode, int capacity,
                            float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out,
                            int32_t* n_admitted_out, double* theta_out,
                            void* stream);

/* ------------------------------------------------------------------------ *
 * Asynchronous capacity.  DSpark paper section 5.2 (the scheduler run
 * asynchronously: capacity from the confidences of two steps earlier, fresh
 * candidates ranked and cut to it); "Speculative decoding, from zero to
 * DSpark", section 9.
 *
 * dspark_schedule in TOPK mode with the capacity read from device memory:
 * `capacity` [1] int32 on the device, typically the n_admitted_out of a
 * DSPARK_SCHED_GLOBAL call made two steps earlier, so that a serving loop
 * fixes the next verify batch size without a host synchronisation.  The
 * first min(max(capacity, 0), number of candidates) candidates of the
 * current a are admitted; a negative capacity (e.g. -1 from a call that saw
 * invalid confidences) admits nothing.  All other arguments, outputs, limits,
 * data errors and the workspace are those of dspark_schedule (capacity may
 * be NULL when R == 0).
 * ------------------------------------------------------------------------ */
int dspark_schedule_async(int R, int K, const float* c,
                          const double* sps, int sps_len,
                          const int32_t* capacity,
                          float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out,
                          int32_t* n_admitted_out, double* theta_out,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ *
 * Rejection-sampling verification over the flattened variable-length batch.
 * DSpark paper section 2.1 and section 5.3 (flattened variable-length
 * batch); "Speculative decoding, from zero to DSpark", section 2 and
 * Appendix A1; the five-step verification routine in the glean.smartcoder
 * article on DSpark.
 *
 * Request r owns flat target rows cu_seqlens[r] .. cu_seqlens[r+1]-1 of P
 * (l_r = cu_seqlens[r+1] - cu_seqlens[r] - 1 drafts, then the bonus row).
 * For j = 1..l_r: p_j = softmax(P[cu[r]+j-1] / T),
 * q_j = softmax((D[r,j-1] + W1[x_{j-1}] W2) / T), x_0 = x0[r]; accept x_j iff
 * u(r, j, accept) < p_j(x_j) / q_j(x_j) (q_j(x_j) == 0 accepts).  At the
 * first rejection the correction is drawn from norm(max(0, p_j - q_j)) with
 * u(r, j, resample); if that mass is zero, from p_j.  If all l_r drafts
 * survive the bonus is drawn from p_{l_r+1} with u(r, l_r + 1, resample).
 * Inputs: P [N, V] (p_dtype), cu_seqlens [R+1] int32 with cu[0] = 0 and
 * cu[R] = N; D [R, K, V] (d_dtype) draft base logits; W1/W2/W2f/r/x0 as for
 * the draft (r == 0: no bias; W2f NULL: W2 read column-major); x [R, K] the
 * drafted tokens.
 * The draft's exact probabilities (both [R, K], both unused when T == 0):
 *   q_tok  q_j(x_j) as returned by dspark_markov_draft, or NULL: computed
 *          from D, the bias and the normaliser;
 *   lse_d  the draft rows' log-normalisers as returned by
 *          dspark_markov_draft, or NULL: recomputed from D (plus the bias)
 *          in an extra pass over the judged draft rows (r == 0: one
 *          streaming pass over the rows j <= l_r; r > 0: the draft's fused
 *          bias pass at every position).
 * Outputs: n_acc_out [R] accepted drafts; tok_out [R] the correction or bonus
 * token (emitted sequence: x_1..x_{n_acc}, tok); min_margin_out [R] or NULL:
 * the smallest margin of the request's decisions, i.e. |u - p_j(x_j)/q_j(x_j)|
 * over the accept tests made (j <= min(n_acc + 1, l_r)) and the distance of
 * the final draw's target u * Z from the nearer CDF edge of the drawn token,
 * divided by the total mass Z; when T == 0 the gap between the largest and
 * the second largest target logit of each examined row (ties give 0).
 * Limits: 0 <= R, 1 <= K <= DSPARK_MAX_K, R <= N <= R * (K + 1), P and D each
 * smaller than 4 GiB.
 * Data errors: a request whose cu_seqlens slice is inconsistent (length < 1 or
 * > K + 1, or outside [0, N]) or whose tokens are outside [0, V) gets
 * n_acc = tok = -1 and min_margin = NaN.
 * Workspace: dspark_verify_workspace_bytes(R, K, V, r, N) bytes (enough for
 * NULL q_tok / lse_d and W2f); 256-byte aligned; contents need not be
 * initialised.
 * ------------------------------------------------------------------------ */
size_t dspark_verify_workspace_bytes(int R, int K, int V, int r, int N);
int dspark_verify(int R, int K, int V, float temperature,
                  const void* P, int p_dtype, int N,
                  const int32_t* cu_seqlens,
                  const void* D, int d_dtype,
                  const void* W1, const void* W2, const void* W2f, int r,
                  const int32_t* x0, const int32_t* x,
                  const float* q_tok, const float* lse_d,
                  uint64_t seed, uint64_t step,
                  int32_t* n_acc_out, int32_t* tok_out, float* min_margin_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Analytic acceptance probability per draft position, the confidence head's
 * training label.  DSpark paper section 3.2.1 (Confidence Head: the label is
 * the per-step acceptance rate set by the total variation distance between
 * draft and target distributions); "Speculative decoding, from zero to
 * DSpark", section 2 (the acceptance probability of one position) and
 * Appendix A4.
 *
 *   c_out[r, k] = 1 - 1/2 || q_{r,k} - p_{r,k} ||_1 = sum_v min(q, p)
 *   q_{r,k} = softmax((D[r, k] + W1[x_{r,k-1}] W2) / T),  x_{r,0} = x0[r]
 *   p_{r,k} = softmax(P[r, k] / T)
 * T == 0: c_out = 1 where the first argmax of P[r, k] is x[r, k], else 0.
 *
 * Inputs: P [B, K, V] (p_dtype) target logits, row (r, k) judging draft
 * position k + 1; D [B, K, V] (d_dtype) draft base logits; W1/W2/W2f/r/x0 as
 * for the draft; x [B, K] the drafted tokens and lse_d [B, K] their
 * log-normalisers, as returned by dspark_markov_draft (lse_d unused when
 * T == 0).  Output: c_out [B, K] f32.
 * Limits: 0 <= B, 1 <= K <= DSPARK_MAX_K, P and D each smaller than 4 GiB.
 * Data errors: a position whose previous or own token is outside [0, V) gets
 * NaN.  Workspace: dspark_acceptance_label_workspace_bytes(B, K, V, r) bytes,
 * 256-byte aligned, contents need not be initialised (with r > 0 and W2f
 * NULL it holds a copy of W2 in MFMA fragment order, written by the call, as
 * for the draft; with W2f the size for r = 0 suffices).
 * ------------------------------------------------------------------------ */
size_t dspark_acceptance_label_workspace_bytes(int B, int K, int V, int r);
int dspark_acceptance_label(int B, int K, int V, float temperature,
                            const void* P, int p_dtype,
                            const void* D, int d_dtype,
                            const void* W1, const void* W2, const void* W2f, int r,
                            const int32_t* x0, const int32_t* x,
                            const float* lse_d, float* c_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * The fp16 copy of W2 in MFMA fragment order that the RNN head's bias
 * passes read (DSpark paper section 3.1, RNN head: the output part meets the
 * same W2 as the Markov embedding).  Written into caller memory W2h
 * (W2h_bytes >= dspark_rnn_w2_f16_bytes(V, r) = ceil(V / 64) * 32 KB,
 * 16-byte aligned) from the column-major bf16 W2, r a multiple of 32 in
 * [32, DSPARK_MAX_RANK]; made once, it serves every RNN call on that W2.
 * ------------------------------------------------------------------------ */
size_t dspark_rnn_w2_f16_bytes(int V, int r);
int dspark_rnn_prepare_w2(int V, int r, const void* W2, void* W2h, size_t W2h_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Sequential RNN-head draft.  DSpark paper section 3.1 ("RNN head");
 * "Speculative decoding, from zero to DSpark", section 6.
 *
 * A state s_k in R^r per request, s_0 = 0.  For k = 1..K in order:
 *   z_k = [s_{k-1}; W1[x_{k-1}]; h_k]            (length 2r + d, x_0 = x0[b])
 *   g = sigmoid(W_g z_k), c~ = tanh(W_c z_k), o_k = W_o z_k
 *   s_k = (1 - g) * s_{k-1} + g * c~
 *   x_k = inverse-CDF draw from softmax((U[b,k-1,:] + o_k W2) / T)
 * W_g, W_c, W_o are the row blocks [0, r), [r, 2r), [2r, 3r) of W.  The
 * page gives z_k, the three parts of one projection and s_0 = 0; its update
 * equation is lost, and the GRU-style blend above, with no additive bias, is
 * this library's reading.  The output part o_k takes the place of the Markov
 * embedding in front of W2 (with W_o = [0 | I | 0] the call is
 * dspark_markov_draft).
 * Inputs: U [B, K, V] (u_dtype f32 or bf16); H [B, K, d] bf16 (h_dtype must
 * be DSPARK_BF16), h_k at [b, k-1]; W [3r, 2r + d] bf16 row-major; W1 [V, r]
 * and W2 (column-major r x V) bf16 as for the Markov draft; x0 [B] int32.
 * Outputs: x_out, q_tok_out, lse_out [B, K] as for dspark_markov_draft;
 * o_out [B, K, r] f32, the output parts o_k, which dspark_rnn_verify and
 * dspark_rnn_acceptance_label take to rebuild the draft distributions.
 * The bias o_k W2 runs on the fp16 MFMA with o_k split into hi + lo fp16
 * parts and W2 converted to fp16 (relative error 2^-22 on o_k): entries of
 * o_k and W2 must be smaller than 2^15 in magnitude.  The fp16 copy of W2 is
 * laid out in MFMA fragment order (ceil(V / 64) x 32 KB, which must be
 * smaller than 4 GiB): W2h, made once by dspark_rnn_prepare_w2, or NULL, and
 * each RNN call then makes it in its workspace.
 * Limits: 0 <= B, 1 <= K <= DSPARK_MAX_K, 1 <= V, r a multiple of 32 in
 * [32, DSPARK_MAX_RANK], d a positive multiple of 64; U, H, W, W1 each smaller
 * than 4 GiB; H, W, W1, W2, o_out 16-byte aligned (else DSPARK_E_RANGE).
 * Workspace: dspark_rnn_draft_workspace_bytes(B, K, V, r, d) bytes.
 * Data errors: an anchor (or the previous drawn token) outside [0, V) makes
 * that request's remaining positions x = -1, q_tok = lse = NaN.
 * ------------------------------------------------------------------------ */
size_t dspark_rnn_draft_workspace_bytes(int B, int K, int V, int r, int d);
int dspark_rnn_draft(int B, int K, int V, int r, int d, float temperature,
                     const void* U, int u_dtype,
                     const void* H, int h_dtype,
                     const void* W, const void* W1, const void* W2, const void* W2h,
                     const int32_t* x0,
                     uint64_t seed, uint64_t step,
                     int32_t* x_out, float* q_tok_out, float* lse_out, float* o_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Verification of RNN-head drafts: dspark_verify with the draft rows'
 * bias rebuilt from the head's output parts, q_j = softmax((D[r,j-1] +
 * O[r,j-1] W2) / T - lse_d) (DSpark paper section 3.1, RNN head, and the
 * sources cited for dspark_verify).  O [R, K, r] f32 as returned in o_out by
 * dspark_rnn_draft (16-byte aligned); W2 column-major bf16; W2h as for
 * dspark_rnn_draft; r as for dspark_rnn_draft.  q_tok and lse_d are required
 * when T > 0 (the draft returns them).  Workspace:
 * dspark_rnn_verify_workspace_bytes(R, K, V, r, N) bytes (dspark_verify's,
 * plus an fp16 copy of W2 unless W2h is given).  Everything else is as for
 * dspark_verify.
 * ------------------------------------------------------------------------ */
size_t dspark_rnn_verify_workspace_bytes(int R, int K, int V, int r, int N);
int dspark_rnn_verify(int R, int K, int V, float temperature,
                      const void* P, int p_dtype, int N,
                      const int32_t* cu_seqlens,
                      const void* D, int d_dtype,
                      const float* O, const void* W2, const void* W2h, int r,
                      const int32_t* x0, const int32_t* x,
                      const float* q_tok, const float* lse_d,
                      uint64_t seed, uint64_t step,
                      int32_t* n_acc_out, int32_t* tok_out, float* min_margin_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Acceptance label of RNN-head drafts: dspark_acceptance_label with
 * q_{r,k} = softmax((D[r,k] + O[r,k] W2) / T) (DSpark paper sections 3.1 and
 * 3.2.1).  O [B, K, r] f32 from dspark_rnn_draft; W2h as for
 * dspark_rnn_draft; workspace: dspark_rnn_acceptance_label_workspace_bytes(B,
 * K, V, r) bytes; otherwise as for dspark_acceptance_label.
 * ------------------------------------------------------------------------ */
size_t dspark_rnn_acceptance_label_workspace_bytes(int B, int K, int V, int r);
int dspark_rnn_acceptance_label(int B, int K, int V, float temperature,
                                const void* P, int p_dtype,
                                const void* D, int d_dtype,
                                const float* O, const void* W2, const void* W2h, int r,
                                const int32_t* x0, const int32_t* x,
                                const float* lse_d, float* c_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Confidence head.  DSpark paper section 3.2.1 (Confidence Head: a linear
 * projection of the backbone hidden state and the Markov embedding of the
 * previous token, then a sigmoid; Post-hoc Calibration: one temperature per
 * position); "Speculative decoding, from zero to DSpark", section 8 (The
 * confidence head).
 *
 *   z[r, k] = w_h . H[r, k] + w_e . W1[x_{r,k-1}] + bias,  x_{r,0} = x0[r]
 *   c_out[r, k] = sigmoid(z[r, k] / T_k)
 * Inputs: H [B, K, d] (h_dtype) hidden states; w_h [d] f32; w_e [r] f32 and
 * W1 [V, r] bf16 (unused when r == 0); x0 [B], x [B, K] int32 (the drafted
 * tokens; x[r, K-1] is not used); sts_temperature [K] f32 from dspark_sts_fit,
 * or NULL for T_k = 1.  Outputs: c_out [B, K] f32, the scheduler's c;
 * logit_out [B, K] f32 (z, for calibration data) or NULL.
 * Limits: 0 <= B, 1 <= K <= DSPARK_MAX_K, d >= 1, H smaller than 4 GiB.
 * Data errors: a previous token outside [0, V) gives NaN.  No workspace.
 * ------------------------------------------------------------------------ */
int dspark_confidence_head(int B, int K, int V, int d, int r,
                           const void* H, int h_dtype,
                           const float* w_h, const float* w_e, float bias,
                           const void* W1, const int32_t* x0, const int32_t* x,
                           const float* sts_temperature,
                           float* c_out, float* logit_out, void* stream);

/* ------------------------------------------------------------------------ *
 * Sequential Temperature Scaling.  DSpark paper section 3.2.1 (Post-hoc
 * Calibration); "Speculative decoding, from zero to DSpark", Appendix A5.
 *
 * On held-out data, left to right over k = 1..K: T_out[k] is the first value
 * of grid minimising the expected calibration error of the cumulative
 * product prod_{i<=k} sigmoid(logits[n, i] / T_i) against survived[n, k]
 * (1 where positions 1..k were all accepted), T_1..T_{k-1} already fixed.
 * ECE: n_bins equal-width bins on [0, 1] (last one closed), sum over bins of
 * |labels - predictions| / N; products and sums in fp64, reduced in a fixed
 * order (deterministic).  A sample whose logit is NaN (dspark_confidence_head
 * reports NaN for an invalid token) has no prediction from that position on:
 * it falls in no bin but still counts in N.
 * Inputs (device): logits [N, K] f32 (logit_out of dspark_confidence_head on
 * held-out requests), survived [N, K] uint8, grid [n_grid] f32 (> 0).
 * Outputs (device): T_out [K] f32; ece_out [K] f32 (the ECE at the chosen
 * temperature) or NULL.
 * Limits: N >= 1, 1 <= K <= DSPARK_MAX_K, 1 <= n_grid <= DSPARK_STS_MAX_GRID,
 * 1 <= n_bins <= DSPARK_STS_MAX_BINS.  Workspace:
 * dspark_sts_fit_workspace_bytes(N, K, n_grid) bytes (a 16-byte record per
 * sample holding its fp64 cumulative product, and per-bin partials of each
 * grid temperature over chunks of 4096 samples; about
 * 16 N + 12 * 32 * n_grid * ceil(N / 4096)).
 * ------------------------------------------------------------------------ */
size_t dspark_sts_fit_workspace_bytes(int N, int K, int n_grid);
int dspark_sts_fit(int N, int K, const float* logits, const uint8_t* survived,
                   int n_grid, const float* grid, int n_bins,
                   float* T_out, float* ece_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * The per-decision uniforms themselves (the seeded counter-based stream the
 * three calls consume): out[i] = u(seed, step, request i, position, purpose)
 * for i in [0, n).  Limits: n >= 0, 0 <= position < 2^30, purpose in {0, 1, 2}.
 * ------------------------------------------------------------------------ */
int dspark_uniforms(uint64_t seed, uint64_t step, int n, int position, int purpose, float* out,
                    void* stream);

/* ------------------------------------------------------------------------ *
 * Kernel timing (instrumentation, not part of the method).  While enabled,
 * every kernel the calls above launch carries a start and a stop HIP event
 * that the dispatch itself records around the kernel's execution
 * (hipExtLaunchKernel), so no extra packets enter the caller's stream and
 * the times match a kernel trace.  dspark_profiler_read waits for the
 * recorded events and reports, per kernel name, the number of launches and the
 * summed event time.  Host-side state shared by every thread of the process
 * (calls from several threads are safe); a name returned by
 * dspark_profiler_read stays valid until the next dspark_profiler_reset.
 * ------------------------------------------------------------------------ */
int dspark_profiler_enable(int on);
int dspark_profiler_reset(void);
/* index in [0, count); returns the number of distinct kernels when name == NULL. */
int dspark_profiler_read(int index, const char** name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
