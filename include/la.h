/*
 * la.h -- C ABI of the MI355X (gfx950) linear-attention library, liblinattn.so.
 *
 * Linear attention with the feature map phi(x) = elu(x) + 1 (ELU slope 1):
 * phi(x) = x + 1 for x > 0 and exp(x) otherwise.  Sources, by page and section
 * ("Transformers are RNNs" blog digest by irregular6612, the velog review
 * "[논문 리뷰] Transformers are RNNs", and the itwiki article "선형 어텐션"):
 *   - feature map and kernelised similarity sim(q,k) = phi(q).phi(k): blog
 *     digest "Methods"; velog 3.2-3.3; itwiki "Formulas";
 *   - non-causal form phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1): blog digest
 *     "Method / key components 2)"; velog 3.2; itwiki "reordering by
 *     associativity";
 *   - causal prefix sums S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i}
 *     phi(k_j), out_i = phi(q_i)^T S_i / phi(q_i)^T z_i: blog digest
 *     "key components 3)"; velog 3.4; itwiki "Causal masking and the
 *     recurrent form";
 *   - chunked evaluation (matrix products inside a chunk, state carried
 *     between chunks): itwiki table "Comparison of forms" and the remark that
 *     training kernels use the chunked form;
 *   - recurrent step S += phi(k) v^T, z += phi(k), then read: blog digest
 *     "key components 4)"; velog 3.6; itwiki "Causal masking and the
 *     recurrent form";
 *   - gradient as cumulative sums with linear memory: velog 3.5; blog digest
 *     "Methods" (last item);
 *   - fixed per-head decay of the state: itwiki, table of later variants,
 *     RetNet row (la_fwd_causal_decay, la_bwd_causal_decay,
 *     la_decode_step_decay);
 *   - choice of feature map (elu + 1, Performer's positive random features,
 *     identity): itwiki section "특징 사상 선택"; blog digest "Digest"
 *     (the *_fm entry points).
 *
 * Conventions shared by every entry point
 *   Layout    All tensors are dense, row-major and contiguous:
 *             sequences [B][H][N][d], state S [B][H][d_k][d_v],
 *             normaliser z [B][H][d_k], per-token denominators [B][H][N],
 *             per-step decode vectors [B][H][d], per-head decays [H].
 *             Every tensor pointer must be 16-byte aligned (gamma: 4-byte).
 *   Sizes     d_k, d_v in {16, 32, 64, 128}, chosen independently;
 *             1 <= N <= 2^30 (LA_ERR_BAD_SHAPE beyond; the workspace queries
 *             return 0), N need not be a multiple of C; C in {16, 32, 64};
 *             B, H >= 1.
 *   Dtypes    `in` is the storage type of q, k, v (and dO, dq, dk, dv);
 *             `out` that of o.  S, z and den are always fp32.  Arithmetic is
 *             fp32 accumulate; for LA_BF16 inputs the matrix products take
 *             bf16 operands (MFMA), for LA_F32 inputs they stay in fp32.
 *   Ownership The caller allocates every buffer, including the workspace
 *             (size from the matching *_workspace_bytes query); the library
 *             allocates nothing and keeps no state between calls.
 *   Streams   Every call only enqueues work on `stream` (0 = the null stream)
 *             and returns; results are ready when the stream has reached it.
 *   Errors    All arguments are checked before anything is enqueued; a bad
 *             argument returns a non-zero la_status and launches nothing.  A
 *             failed launch returns LA_ERR_LAUNCH.  No C++ exception crosses
 *             the ABI.
 *   Non-finite values are propagated, not reported.  In the causal forward a
 *             NaN or +Inf in q at token i makes out_i (and den_i) non-finite
 *             and nothing else; in k or v at token j it makes every output at
 *             and after j of that (b, h) non-finite, leaves every output
 *             before the C-token chunk holding j unchanged, and may reach the
 *             earlier tokens of that chunk (a masked product with a zero
 *             weight still carries a NaN).  -Inf in k is phi = 0: a token
 *             without weight.  The non-causal form spreads a non-finite k or v
 *             to every output of its (b, h); the decode step spreads a
 *             non-finite k or v into S and z, and so into every later step.
 *             Other (b, h) pairs are never affected.
 *   Underflow No denominator epsilon is added: phi(x) = exp(x) underflows to 0
 *             in fp32 below about -87 (-104 with subnormals), so a query whose
 *             entries all lie below that has den = 0 and a non-finite output,
 *             as the formulas imply.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL_PTR = 1,     /* a required pointer is NULL                       */
    LA_ERR_BAD_SHAPE = 2,    /* B, H or N out of range                           */
    LA_ERR_UNSUPPORTED = 3,  /* d_k, d_v or C outside the supported sets         */
    LA_ERR_BAD_DTYPE = 4,    /* unknown la_dtype value                           */
    LA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the query says    */
    LA_ERR_LAUNCH = 6,       /* the HIP runtime rejected a launch                */
    LA_ERR_ALIGNMENT = 7     /* a pointer is not 16-byte aligned                 */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Feature map phi of the *_fm entry points (itwiki "선형 어텐션", section
 * "특징 사상 선택" (choice of feature map), which lists these three):
 *   LA_PHI_ELU1      phi = elu + 1, as every other entry point (W, m unused);
 *   LA_PHI_IDENTITY  phi(x) = x: q and k already are the features (W, m
 *                    unused).  The normaliser phi(q) . sum phi(k) must stay
 *                    away from zero; nothing checks it;
 *   LA_PHI_PRF       Performer's positive random features, an unbiased
 *                    estimate of the softmax kernel exp(q . k):
 *                    phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), r < m,
 *                    with W [H][m][d_k] in the input type holding m directions
 *                    w_r per head (drawn by the caller, e.g. from N(0, I) in
 *                    orthogonal blocks), d_k and m in {32, 64, 128}.  The
 *                    features stay in fp32 range while |x|^2 / 2 - w_r . x
 *                    stays below about 87.  The state then has m rows:
 *                    S [B][H][m][d_v], z [B][H][m]. */
typedef enum { LA_PHI_ELU1 = 0, LA_PHI_IDENTITY = 1, LA_PHI_PRF = 2 } la_feature_map;

/* Human-readable text for a status code (static storage, never NULL). */
const char *la_status_string(la_status s);

/* Workspace bytes each entry point needs for these sizes (0 is a valid
 * answer: then `ws` may be NULL).  Invalid sizes return 0; the entry point
 * itself reports the error. */
size_t la_fwd_causal_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C);
size_t la_fwd_noncausal_workspace_bytes(int B, int H, int N, int d_k, int d_v);
size_t la_bwd_causal_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C);
size_t la_bwd_noncausal_workspace_bytes(int B, int H, int N, int d_k, int d_v);

/*
 * Non-causal forward: o_i = phi(q_i)^T (sum_j phi(k_j) v_j^T) /
 *                           phi(q_i)^T (sum_j phi(k_j)),  sums over all N.
 * q, k: [B][H][N][d_k] (in); v: [B][H][N][d_v] (in); o: [B][H][N][d_v] (out).
 */
la_status la_fwd_noncausal(const void *q, const void *k, const void *v, void *o,
                           int B, int H, int N, int d_k, int d_v,
                           la_dtype in, la_dtype out,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Causal forward, evaluated chunk by chunk (C tokens per chunk):
 *   o_i = phi(q_i)^T S_i / den_i,  den_i = phi(q_i)^T z_i,
 *   S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j).
 * The result does not depend on C (the chunked form is an exact rewrite);
 * C only sets the tiling.  den (nullable, fp32 [B][H][N]) receives den_i.
 */
la_status la_fwd_causal(const void *q, const void *k, const void *v, void *o, float *den,
                        int B, int H, int N, int d_k, int d_v, int C,
                        la_dtype in, la_dtype out,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Causal forward with a carried state (prefill that hands over to decode):
 * as la_fwd_causal, but the prefix sums start from S0, z0 instead of zero
 * (S0 [B][H][d_k][d_v], z0 [B][H][d_k], fp32, both NULL for a zero start),
 * and the state after the last token is written to S_out, z_out (fp32, both
 * NULL to skip).  S_out/z_out may alias S0/z0.  With S_out, z_out from one
 * call passed as S0, z0 to the next, two calls over the halves of a sequence
 * give the same outputs as one call over the whole, and S_out, z_out seed
 * la_decode_step.
 */
la_status la_fwd_causal_state(const void *q, const void *k, const void *v, void *o, float *den,
                              const float *S0, const float *z0, float *S_out, float *z_out,
                              int B, int H, int N, int d_k, int d_v, int C,
                              la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Causal forward with a fixed per-head decay (itwiki "선형 어텐션", table of
 * later variants, RetNet row, S_t = gamma S_{t-1} + ...), keeping the feature
 * map and the normaliser of the base method:
 *   S_i = gamma_h S_{i-1} + phi(k_i) v_i^T,  z_i = gamma_h z_{i-1} + phi(k_i),
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
 * gamma: device pointer to H fp32 values, gamma_h for head h, each in
 * [0, 1] (gamma = 0 keeps only the current token: out_i = v_i).  The chunked
 * evaluation applies only powers gamma^e with e >= 0, so every value in the
 * range is exact to rounding.  A NULL gamma is no decay (la_fwd_causal_state).  S0, z0 enter decayed like any earlier state; S_out,
 * z_out receive the decayed state after the last token and seed
 * la_decode_step_decay.  Other arguments, the workspace (the query of
 * la_fwd_causal) and errors as la_fwd_causal_state.
 */
la_status la_fwd_causal_decay(const void *q, const void *k, const void *v, void *o, float *den,
                              const float *S0, const float *z0, float *S_out, float *z_out, const float *gamma,
                              int B, int H, int N, int d_k, int d_v, int C,
                              la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Causal forward that allocates nothing, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, result and errors as la_fwd_causal, without
 * the workspace: the per-segment states live in a device array the library
 * owns, LA_NOALLOC_SCRATCH_BYTES per GPU, held from load until the process
 * ends.  The split of each sequence into segments is capped so that its states
 * fit the array (at one segment per (b, h) none are stored, so no size is
 * refused for lack of room; large d_k x d_v problems may run fewer segments
 * than la_fwd_causal and round differently within the usual tolerance).
 * Calls share their GPU's array: calls that overlap on one GPU (other streams
 * or host threads) race and must be serialised by the caller.  The first call
 * on a device looks up the array's address there (hipGetSymbolAddress) and
 * can fail with LA_ERR_LAUNCH.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
la_status la_fwd_causal_noalloc(const void *q, const void *k, const void *v, void *o, float *den,
                                int B, int H, int N, int d_k, int d_v, int C,
                                la_dtype in, la_dtype out, hipStream_t stream);

/*
 * Causal backward by cumulative sums: the exact gradient of la_fwd_causal
 * with respect to q, k and v for an upstream gradient dO.
 * With g_i = dO_i, den_i = phi(q_i) . z_i, gh_i = g_i / den_i and
 * eps_i = -(g_i . o_i) / den_i:
 *   dphi(q_i) = S_i gh_i + eps_i z_i                   (forward prefix sums)
 *   dphi(k_j) = R_j v_j + r_j,  dv_j = R_j^T phi(k_j)  (reverse suffix sums)
 *   with R_j = sum_{i>=j} phi(q_i) gh_i^T, r_j = sum_{i>=j} phi(q_i) eps_i,
 *   then dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k).
 * The forward's outputs are not inputs: den_i and the products with o_i are
 * recomputed from the prefix sums inside the dq sweep.
 * Inputs q, k [B][H][N][d_k], v, dO [B][H][N][d_v] in `in`; outputs dq, dk
 * [B][H][N][d_k] and dv [B][H][N][d_v] in `in`.  No per-token state is
 * stored: the workspace (always required) holds two floats per token and
 * per-segment d_k x (d_v + 1) prefix and suffix sums.
 */
la_status la_bwd_causal(const void *q, const void *k, const void *v, const void *dO,
                        void *dq, void *dk, void *dv,
                        int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of la_fwd_causal_decay (itwiki "선형 어텐션", table of later
 * variants, RetNet row; the gradient as cumulative sums with linear memory,
 * velog 3.5): the exact gradient with respect to q, k and v of the decayed
 * causal form with zero initial state.  It is the gradient of la_bwd_causal
 * with every pair (i, j <= i) weighed by gamma_h^(i - j):
 *   dphi(q_i) = S_i gh_i + eps_i z_i        (decayed prefix sums S_i, z_i)
 *   dphi(k_j) = R_j v_j + r_j,  dv_j = R_j^T phi(k_j),
 *   R_j = sum_{i>=j} gamma^(i - j) phi(q_i) gh_i^T,  r_j likewise with eps_i.
 * gamma: device pointer to H fp32 values in [0, 1] (NULL returns
 * LA_ERR_NULL_PTR).  Other arguments, the workspace (the query of
 * la_bwd_causal) and errors as la_bwd_causal.
 */
la_status la_bwd_causal_decay(const void *q, const void *k, const void *v, const void *dO,
                              void *dq, void *dk, void *dv, const float *gamma,
                              int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the non-causal form (blog digest "Method / key components 2)";
 * velog 3.2 for the form, 3.5 for the gradient as sums with linear memory):
 * the exact gradient of la_fwd_noncausal with respect to q, k and v for an
 * upstream gradient dO.  The formulas are those of la_bwd_causal with the
 * prefix and suffix sums replaced by full sums over all N tokens:
 *   dphi(q_i) = S gh_i + eps_i z,  S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j)
 *   dphi(k_j) = R v_j + r,  dv_j = R^T phi(k_j),
 *   R = sum_i phi(q_i) gh_i^T, r = sum_i phi(q_i) eps_i,
 * then dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k).  Layouts, dtypes and
 * errors as la_bwd_causal; there is no C argument (the tiling is internal).
 * The workspace (always required) holds two floats per token and
 * per-segment d_k x (d_v + 1) partial sums.
 */
la_status la_bwd_noncausal(const void *q, const void *k, const void *v, const void *dO,
                           void *dq, void *dk, void *dv,
                           int B, int H, int N, int d_k, int d_v, la_dtype in,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The causal forward, the non-causal forward, the causal backward and the
 * decode step with a feature map (la_feature_map above).  Arguments, layouts
 * and errors are those of the plain entry points, plus fm, W and m; the
 * workspace queries take them and the input type too.  Random features are
 * computed on the matrix cores.  The forwards with bf16 inputs, m = d_k in
 * {32, 64}, d_v <= 64 and C = 64 (every non-causal call of such a shape) form them in the
 * chunked kernels as q and k are loaded, so the workspace is that of the
 * plain forward; other shapes first write phi(q), phi(k) to the workspace as
 * [B][H][N][m] in the input type and run the chunked kernels with the
 * identity map over m features.  The backward keeps phi(q), phi(k), dphi(q),
 * dphi(k) in the workspace in fp32 and carries dphi back through the map:
 * dx = sum_r dphi_r phi_r(x) (w_r - x); its cumulative sums multiply fp32
 * operands for LA_F32 inputs and, for LA_BF16 inputs, operands held as a bf16
 * value plus its bf16 remainder (about 16 bits).  An unknown fm, or m or d_k outside
 * {32, 64, 128} with LA_PHI_PRF, returns LA_ERR_UNSUPPORTED; a NULL W with
 * LA_PHI_PRF returns LA_ERR_NULL_PTR.
 */
size_t la_fwd_causal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C,
                                        la_feature_map fm, int m, la_dtype in);
size_t la_fwd_noncausal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v,
                                           la_feature_map fm, int m, la_dtype in);
size_t la_bwd_causal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C,
                                        la_feature_map fm, int m, la_dtype in);
la_status la_fwd_causal_fm(const void *q, const void *k, const void *v, void *o, float *den,
                           la_feature_map fm, const void *W, int m,
                           int B, int H, int N, int d_k, int d_v, int C, la_dtype in, la_dtype out,
                           void *ws, size_t ws_bytes, hipStream_t stream);
la_status la_fwd_noncausal_fm(const void *q, const void *k, const void *v, void *o,
                              la_feature_map fm, const void *W, int m,
                              int B, int H, int N, int d_k, int d_v, la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream);
la_status la_bwd_causal_fm(const void *q, const void *k, const void *v, const void *dO,
                           void *dq, void *dk, void *dv, la_feature_map fm, const void *W, int m,
                           int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                           void *ws, size_t ws_bytes, hipStream_t stream);
/* S [B][H][m'][d_v], z [B][H][m'] with m' = m for LA_PHI_PRF, d_k otherwise. */
la_status la_decode_step_fm(float *S, float *z, const void *q, const void *k, const void *v, void *o,
                            la_feature_map fm, const void *W, int m,
                            int B, int H, int d_k, int d_v, la_dtype in, hipStream_t stream);

/*
 * One recurrent decode step for every (b, h):
 *   S += phi(k) v^T;  z += phi(k);  o = phi(q)^T S / (phi(q) . z)
 * (update first, then read).  S [B][H][d_k][d_v] and z [B][H][d_k] are fp32,
 * read and written in place; the caller zeroes them before the first step.
 * q, k: [B][H][d_k], v: [B][H][d_v] and o: [B][H][d_v] in `in`.
 */
la_status la_decode_step(float *S, float *z, const void *q, const void *k, const void *v,
                         void *o, int B, int H, int d_k, int d_v, la_dtype in,
                         hipStream_t stream);

/*
 * Decode step with a fixed per-head decay (itwiki "선형 어텐션", table of
 * later variants, RetNet row, S_t = gamma S_{t-1} + ...; the feature map and
 * the normaliser of the base method are kept):
 *   S = gamma_h S + phi(k) v^T;  z = gamma_h z + phi(k);  o = phi(q)^T S / (phi(q) . z)
 * gamma: device pointer to H fp32 values, gamma_h for head h (values in
 * [0, 1]; 1 gives la_decode_step).  Other arguments as la_decode_step; a
 * NULL gamma returns LA_ERR_NULL_PTR.
 */
la_status la_decode_step_decay(float *S, float *z, const void *q, const void *k, const void *v,
                               void *o, const float *gamma, int B, int H, int d_k, int d_v, la_dtype in,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
