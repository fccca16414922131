/*
 * plx.h -- C ABI of the Parallax attention library for AMD MI355X (gfx950).
 *
 * The operator (parameterized Local Linear Attention, boundary factor eta = 0):
 *
 *     o_i = o_i^SA - Sigma_KV^(i) rho_i
 *
 *   o^SA          causal softmax attention with scale tau (usually 1/sqrt(d));
 *   Sigma_KV^(i)  sum_j w_ij (v_j - vbar_i)(k_j - kbar_i)^T, the softmax-weighted
 *                 KV covariance, w_ij = softmax_j(tau q_i . k_j),
 *                 vbar_i = sum_j w_ij v_j, kbar_i = sum_j w_ij k_j;
 *   rho_i         the per-token probe (a learned projection W_R x_i computed by
 *                 the caller, outside this library).
 *
 * Sources: "当注意力学会追问：Parallax如何给Transformer装上第二只眼" (zhichai.net),
 * section 1.3, formula o_i^PLX = o_i^SA - Sigma_KV^(i) rho_i with rho_i = W_R x_i;
 * "Riepilogo Tecnico: Parallax ..." (gist.science), section "Meccanismo
 * Principale" (same formula; eta_i set to zero) and section "Algoritmo
 * Consapevole dell'Hardware" (one streaming pass reusing the KV stream, QK and
 * RK in the same matrix instructions, a custom decode kernel).  The pages call
 * Sigma_KV only "the KV covariance"; the explicit weighted form above is the
 * reading this library implements.
 *
 * Conventions shared by every entry point
 *   - Layout: dense, contiguous [B, H, T, d] (d fastest).  K and V use Hkv heads,
 *     q / rho / dO use Hq heads; query head h reads KV head h / (Hq / Hkv).
 *   - dtype applies to q, k, v, rho and dO: PLX_BF16 (bf16 storage; score GEMMs in
 *     bf16 MFMA with fp32 accumulation, softmax-weighted GEMMs with fp16 operands
 *     and fp32 accumulation) or PLX_F32 (fp32 throughout).  Every output (o, LSE,
 *     auxiliaries, gradients) is fp32.
 *   - bf16 inputs that feed fp16 operands (v in every call; q, rho, dO and k as
 *     well in plx_bwd) must lie within fp16's range, |x| <= 65504: the
 *     conversion is exact down to 2^-14 and rounds smaller magnitudes to fp16's
 *     subnormal grid (absolute error <= 2^-25); larger ones become infinite.
 *   - bf16 probe scores: the forward and decode kernels round p * r (p <= 16,
 *     the softmax numerator against a running maximum that moves only when a
 *     score exceeds it by more than 4 in log2 units) to fp16, so every probe
 *     score must satisfy |r_ij| = |rho_i . k_j| <= 4094 (fp16's largest
 *     value over 16).  The workloads' probes give |r| of a few tens.
 *   - Supported head dims: d = 64 or 128 (d_k = d_v = d) everywhere; d = 256 as
 *     well for every bf16 call (PLX_ERR_UNSUPPORTED for fp32 at d = 256).
 *   - All pointers are DEVICE pointers unless stated.  The caller owns every
 *     buffer; the library never allocates or frees device memory and keeps no
 *     state between calls.  Calls are asynchronous on `stream` (a hipStream_t;
 *     NULL is the default stream); device faults surface at the caller's sync.
 *   - Errors: arguments are validated before any HIP call.  Bad pointers / sizes
 *     return PLX_ERR_INVALID_ARG, valid but unsupported shapes return
 *     PLX_ERR_UNSUPPORTED, a short workspace returns PLX_ERR_WORKSPACE, a failed
 *     launch returns PLX_ERR_HIP.  Nothing is launched when an error is returned.
 *   - Thread-safe: no global mutable state.
 */
#ifndef PLX_H_
#define PLX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PLX_OK = 0,
  PLX_ERR_INVALID_ARG = 1,
  PLX_ERR_UNSUPPORTED = 2,
  PLX_ERR_WORKSPACE = 3,
  PLX_ERR_HIP = 4
} plx_status;

typedef enum { PLX_F32 = 0, PLX_BF16 = 1 } plx_dtype;

/* Opaque stream handle; pass a hipStream_t (or NULL for the default stream). */
typedef void* plx_stream;

/* ABI version of this header (incremented on incompatible changes). */
#define PLX_ABI_VERSION 1
int plx_abi_version(void);

/* Static text for a status code (never NULL). */
const char* plx_status_string(plx_status s);

/*
 * Causal prefill forward.
 *
 * Computes, for every (b, h, i) with keys j <= i (diagonal included),
 *   o[b,h,i,:] = vbar_i - Sigma_KV^(i) rho_i  (fp32),
 * in one streaming pass that carries the online-softmax max and sum with the
 * accumulators O = P V, U = (P . R) V and C = rowsum(P . R), R = rho K^T, and
 * ends with o = (O/l)(1 + C/l) - U/l (the identity
 * Sigma_KV rho = sum_j w_j (k_j . rho) v_j - vbar (kbar . rho)).
 *
 *   q, rho      [B, Hq, T, d]   dtype
 *   k, v        [B, Hkv, T, d]  dtype
 *   o           [B, Hq, T, d]   fp32, written
 *   lse         [B, Hq, T]      fp32 natural log-sum-exp of tau q.k, or NULL
 *   c_aux       [B, Hq, T]      fp32 c_i = kbar_i . rho_i, or NULL
 *   vbar_aux    [B, Hq, T, d]   fp32 vbar_i (the softmax-attention output), or NULL
 *   scale       tau > 0 (finite)
 * lse, c_aux and vbar_aux are the auxiliaries plx_bwd needs.
 * Requires B, Hq, Hkv, T >= 1, Hq % Hkv == 0, d in {64, 128} (or 256, bf16), 16-byte aligned
 * pointers.  A T that is not a multiple of any tile size is handled exactly.
 */
plx_status plx_fwd_prefill(const void* q, const void* k, const void* v, const void* rho,
                           float* o, float* lse, float* c_aux, float* vbar_aux,
                           int B, int Hq, int Hkv, int T, int d, float scale,
                           plx_dtype dtype, plx_stream stream);

/*
 * Decode: one new query and probe per (b, h) against a KV cache.
 *
 * The pages describe a custom decode kernel that streams the KV cache once
 * for both branches ("Riepilogo Tecnico: Parallax ..." (gist.science),
 * section "Algoritmo Consapevole dell'Hardware") and a variant tuned for
 * parallel decoding ("Внимание нового поколения ..." (denisavetisyan.com),
 * the decode-latency figure); the key split below is that parallelism.  The
 * output is the operator above at the query's position, with the cache rows
 * as its key set.
 *
 * Query (b, h) attends to the cache rows [0, ctx_len[b]) of KV head h/(Hq/Hkv)
 * (the cache already holds the current token; no mask).  The keys are cut into
 * ranges processed by separate workgroups, each producing a partial record
 * (m, l, e, C, O, U) -- running max, sum of P as the value GEMMs used it, sum
 * of the unrounded p, sum of P . R, P V and (P . R) V -- which a second kernel
 * merges:
 *   M = max m_s, a_s = exp(m_s - M), l = sum a_s l_s, e/C/O/U likewise,
 *   o = (O/l)(1 + C/l) - U/l,   LSE = M + ln e.
 * C/l equals kbar . rho (kbar = P K / l), the only use the output makes of the
 * mean key, so the record carries that scalar instead of the vector P K.
 *
 * num_splits = 0 (bf16): the (b, kv head, key) space of all sequences, laid end
 * to end, is cut into equal contiguous ranges, one per workgroup (at most 512,
 * two per compute unit), so ragged lengths keep every workgroup equally busy.
 * num_splits > 0, or fp32: every sequence's [0, S_max) is cut into num_splits
 * equal splits (fp32 with 0 picks the count automatically).
 *
 *   q, rho        [B, Hq, d]          dtype
 *   k_cache       [B, Hkv, S_max, d]  dtype
 *   v_cache       [B, Hkv, S_max, d]  dtype
 *   ctx_len       [B] int32, DEVICE memory, read by the kernels.  A value outside
 *                 [1, S_max] makes that sequence's o and lse NaN (no out-of-range
 *                 cache row is ever read).
 *   o             [B, Hq, d] fp32, written
 *   lse           [B, Hq] fp32, or NULL
 *   num_splits    0 = automatic (see above), else the number of key splits over S_max
 *   workspace     device scratch of at least plx_decode_workspace_size(...) bytes,
 *                 16-byte aligned; contents on entry are ignored
 * Any group size Hq / Hkv: up to 16 query heads of a KV head share one pass
 * over its cache; larger groups take one pass per 16 heads.  Rows of the cache
 * at or beyond ctx_len[b] are never read.  The result is deterministic (no atomics; the
 * waves of a workgroup and the records of a head are combined in fixed order).
 */
size_t plx_decode_workspace_size(int B, int Hq, int Hkv, int S_max, int d, int num_splits);
plx_status plx_decode(const void* q, const void* rho, const void* k_cache, const void* v_cache,
                      const int32_t* ctx_len, float* o, float* lse,
                      int B, int Hq, int Hkv, int S_max, int d, float scale, int num_splits,
                      void* workspace, size_t workspace_bytes, plx_dtype dtype, plx_stream stream);

/*
 * Decode with no workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It computes exactly what plx_decode computes (same
 * kernels, same schedule, bitwise the same results) and takes the same
 * arguments less the workspace.  The partial records go to a buffer inside the
 * library instead: one static device array of PLX_DECODE_SCRATCH_BYTES per GPU,
 * whose address is resolved on the first call made with that GPU current and
 * which that GPU holds until the process ends.  The call allocates and frees
 * nothing.
 *   Size limit: plx_decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits) must
 *   not exceed PLX_DECODE_SCRATCH_BYTES; larger problems return
 *   PLX_ERR_WORKSPACE before anything is launched (use plx_decode with a
 *   caller-owned workspace for them).
 *   Sharing: every call on one GPU uses that GPU's single array, which keeps
 *   the last call's records.  Calls whose executions overlap on the same GPU
 *   (different streams, threads or processes' graphs replayed concurrently)
 *   race on it and give wrong results; serialise them, e.g. on one stream.
 */
#define PLX_DECODE_SCRATCH_BYTES (16u << 20)
plx_status plx_decode_noalloc(const void* q, const void* rho, const void* k_cache,
                              const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                              int B, int Hq, int Hkv, int S_max, int d, float scale, int num_splits,
                              plx_dtype dtype, plx_stream stream);

/*
 * Family corners and the correction-to-output ratio.
 *
 * The pages place Parallax in a family of attention operators spanned by three
 * axes ("当注意力学会追问..." (zhichai.net), section 2.1): the bandwidth (softmax
 * weights at a finite temperature, or uniform weights in the h -> infinity
 * limit), the probe, and the affine structure (with an intercept, keeping vbar,
 * or without one, vbar = kbar = 0 as in linear attention).  The _ex entry
 * points take the two switchable axes as flags; flags = 0 is exactly
 * plx_fwd_prefill / plx_decode:
 *   PLX_UNIFORM_WEIGHTS  w_ij = 1/n_i over the key set of query i (the scores
 *                        are not used; the probe scores r_ij still are).  The
 *                        LSE output is then ln n_i.  K must be finite.
 *   PLX_NO_INTERCEPT     vbar = kbar = 0 in the covariance:
 *                        Sigma^(i) = sum_j w_ij v_j k_j^T (uncentred) and
 *                        o_i = -Sigma^(i) rho_i.
 * Both flags together give causal linear attention with query -rho_i and 1/n_i
 * normalisation.
 *
 *   cor   [B, Hq, T] (prefill) or [B, Hq] (decode) fp32, or NULL: the
 *         correction-to-output ratio ||Sigma^(i) rho_i||_2 / ||o_i||_2 per
 *         query, the diagnostic the technical summary ("Riepilogo Tecnico:
 *         Parallax ...", section "Risultati Sperimentali") and "Внимание
 *         нового поколения: локальная линейная модель Parallax ..." (section
 *         "Анализ Parallax: Выводы из внутренних метрик") track; the norms are
 *         read as Euclidean over d.  It is 0 for a single key with an intercept and
 *         1 without an intercept; IEEE inf / NaN when o_i = 0.
 * c_aux and vbar_aux keep their meaning (C/l and O/l, the softmax- or
 * uniformly-weighted means) at every corner; plx_bwd differentiates the
 * flags = 0 operator only.  Every other argument, layout rule and error is as
 * in plx_fwd_prefill / plx_decode; unknown flag bits return PLX_ERR_INVALID_ARG.
 */
#define PLX_UNIFORM_WEIGHTS 1u
#define PLX_NO_INTERCEPT 2u
plx_status plx_fwd_prefill_ex(const void* q, const void* k, const void* v, const void* rho,
                              float* o, float* lse, float* c_aux, float* vbar_aux, float* cor,
                              int B, int Hq, int Hkv, int T, int d, float scale, unsigned flags,
                              plx_dtype dtype, plx_stream stream);
plx_status plx_decode_ex(const void* q, const void* rho, const void* k_cache, const void* v_cache,
                         const int32_t* ctx_len, float* o, float* lse, float* cor, int B, int Hq,
                         int Hkv, int S_max, int d, float scale, int num_splits, unsigned flags,
                         void* workspace, size_t workspace_bytes, plx_dtype dtype,
                         plx_stream stream);

/*
 * The projection in front of the operator.
 *
 * The probe is a learned linear map of the layer input, rho_i = W_R x_i
 * ("当注意力学会追问..." (zhichai.net), section 1.3; "Riepilogo Tecnico:
 * Parallax ...", section "Meccanismo Principale").  With the query, key and
 * value projections it forms one GEMM over the stacked weight
 * W = [W_Q; W_K; W_V; W_R]: for every token, y = W x_t, and the four row
 * blocks of y, split into heads of d rows, are written in the [B, H, T, d]
 * layout the other entry points read.
 *
 *   x      [B, T, D] bf16 (the layer input, tokens of one sequence consecutive)
 *   w      [(2 Hq + 2 Hkv) d, D] bf16: rows [0, Hq d) W_Q, then Hkv d rows of
 *          W_K, Hkv d rows of W_V and Hq d rows of W_R; inside a block, row
 *          h d + j is dimension j of head h
 *   q, rho [B, Hq, T, d] bf16, written;  k, v [B, Hkv, T, d] bf16, written
 * Products accumulate in fp32 and each output is rounded to bf16 (to nearest,
 * ties to even).  Requires dtype = PLX_BF16 (else PLX_ERR_UNSUPPORTED),
 * D % 64 == 0 (else PLX_ERR_UNSUPPORTED), d in {64, 128, 256}, B, T, Hq, Hkv >= 1,
 * Hq % Hkv == 0 and 16-byte aligned pointers.  The outputs must not overlap
 * x or w.
 */
plx_status plx_qkvr_proj(const void* x, const void* w, void* q, void* k, void* v, void* rho,
                         int B, int T, int D, int Hq, int Hkv, int d, plx_dtype dtype,
                         plx_stream stream);

/*
 * Backward of the causal prefill.  The pages give no backward pass; this is
 * the exact gradient of the operator defined by "当注意力学会追问..."
 * (zhichai.net), section 1.3, and "Riepilogo Tecnico: Parallax ..."
 * (gist.science), section "Meccanismo Principale" (o = o^SA - Sigma_KV rho,
 * eta = 0), with rho an independent input, written out in closed form:
 *
 * With g = dO_i, A_ij = g . v_j, G_i = g . o_i, delta_i = g . vbar_i,
 * c_i = kbar_i . rho_i, r_ij = rho_i . k_j and w_ij recomputed from the saved LSE:
 *   dV_j   = sum_i w_ij (1 + c_i - r_ij) g_i
 *   dS_ij  = w_ij [ (1 + c_i - r_ij) A_ij - G_i + delta_i (r_ij - c_i) ]
 *   dR_ij  = -w_ij (A_ij - delta_i)
 *   dQ = tau dS K,  dK = tau dS^T Q + dR^T rho,  drho = dR K.
 * dK and dV sum over the query heads that share a KV head.
 *
 *   q, rho, dO  [B, Hq, T, d]  dtype      k, v  [B, Hkv, T, d]  dtype
 *   o           [B, Hq, T, d]  fp32 (forward output)
 *   lse, c_aux  [B, Hq, T]     fp32 (forward auxiliaries, required)
 *   vbar_aux    [B, Hq, T, d]  fp32 (forward auxiliary, required)
 *   dq, drho    [B, Hq, T, d]  fp32, written (overwritten, not accumulated)
 *   dk, dv      [B, Hkv, T, d] fp32, written (overwritten, not accumulated)
 *   workspace   at least plx_bwd_workspace_size(...) bytes, 16-byte aligned:
 *               G_i and delta_i (fp32 per query row); the dO scale (below) and
 *               the partial maxima it is reduced from; then, used by the bf16
 *               path, fp16 copies of q, rho, s dO ([B, Hq, T, d]) and k
 *               ([B, Hkv, T, d]) that the kernels stage as MFMA operands
 * bf16 path: q, rho, k and v enter fp16 MFMAs (exact for 2^-14 <= |x| <= 65504;
 * smaller magnitudes keep an absolute error of at most 2^-25, larger ones are
 * out of range).  dO enters them scaled by the power of two s with
 * s max|dO| in [1, 2), and the four gradients are multiplied by 1/s as they
 * are stored, so any dO whose gradients fit fp32 (a loss averaged over
 * millions of tokens included) keeps full precision: scaling dO by a power of
 * two scales every gradient by exactly that factor.
 * The result is deterministic (no atomics): one kernel owns each key block and
 * one kernel owns each query block.
 */
size_t plx_bwd_workspace_size(int B, int Hq, int Hkv, int T, int d);
plx_status plx_bwd(const void* q, const void* k, const void* v, const void* rho, const void* d_o,
                   const float* o, const float* lse, const float* c_aux, const float* vbar_aux,
                   float* dq, float* dk, float* dv, float* drho,
                   int B, int Hq, int Hkv, int T, int d, float scale,
                   void* workspace, size_t workspace_bytes, plx_dtype dtype, plx_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* PLX_H_ */
