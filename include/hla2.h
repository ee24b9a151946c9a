/*
 * hla2.h -- C ABI of the MI355X (gfx950) library for strictly causal
 * second-order Higher-order Linear Attention (HLA2).
 *
 * Sources (web pages about arXiv 2510.27258):
 *   [SUM] "Technische Samenvatting: Hogere-orde Lineaire Aandacht (HLA)",
 *         gist.science (technical summary).
 *   [ABS] "Высокоуровневое линейное внимание", chatpaper.ai (abstract).
 *   [SKL] "higher-order-linear-attention-mechanism", skillsmp.com (only its
 *         tensor layout [B, n, H*d] -> [B, H, n, d] is used).
 *
 * Operation, per batch b and head h, tokens t = 0..n-1 (q_t, k_t in R^d,
 * v_t in R^dv):
 *   S_t = sum_{i<=t} g^{t-i} k_i k_i^T        key moment       [SUM §1, state upkeep]
 *   C_t = sum_{i<=t} g^{t-i} q_i v_i^T        query-value acc. [SUM §1, state upkeep]
 *   m_t = sum_{i<=t} g^{t-i} q_i              query mass       [SUM §1, state upkeep]
 *   G_t, h_t: cross summaries holding the pairs (query j < key i) of the
 *             naive product S_t C_t (resp. S_t m_t)             [SUM §1, strict causality]
 *   num_t = q_t^T (S_t C_t - G_t)                               [SUM §1, output]
 *   den_t = q_t^T (S_t m_t - h_t)                               [SUM §1, normalisation]
 *   out_t = num_t, or num_t / den_t when ratio-normalised (IEEE division,
 *           no epsilon).
 * Equivalently num_t = sum_{j<=t} sum_{i<=j} g^{(t-i)+(t-j)} (q_t.k_i)(q_j.k_i) v_j:
 * row t of L o (A A^T) V with A = L o (Q K^T) when g = 1, so out_t depends on
 * tokens j <= t only [SUM "Resultaten en claims"].  g = decay in (0, 1]; the
 * pages name decayed variants without a formula [SUM "Belangrijkste
 * bijdragen" 2]; the reading used is that every first-order summary decays
 * by g per token (g = 1: no decay).
 *
 * The forward pass is computed chunk-parallel [SUM §4]: the sequence is cut
 * into chunks of `chunk` tokens, runs of consecutive chunks are reduced to
 * segment summaries, an exclusive scan with the semidirect-product combine
 * gives every segment its incoming state, and the chunks are walked again
 * from that state to produce the outputs.  The activations equal those of
 * the serial recurrence up to floating-point rounding [SUM §4, scan
 * equivalence].
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    contiguous, row-major, owned by the caller.  The library allocates
 *    nothing on these paths and keeps no state between calls.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *  - Arguments are validated on the host before any device call; an invalid
 *    call returns a negative code and enqueues nothing.  Launch failures are
 *    reported as HLA2_ERR_LAUNCH.  NaN/Inf inputs are not checked; they
 *    propagate.  den = 0 under ratio normalisation gives IEEE +-Inf/NaN.
 *  - Nothing is thrown across the ABI.
 */
#ifndef HLA2_H_
#define HLA2_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out.  Accumulation is always fp32. */
typedef enum { HLA2_F32 = 0, HLA2_BF16 = 1 } hla2_dtype_t;

enum {
  HLA2_OK = 0,
  HLA2_ERR_INVALID = -1,     /* null pointer, size <= 0, decay outside (0,1], ... */
  HLA2_ERR_UNSUPPORTED = -2, /* shape or chunk outside the supported set */
  HLA2_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  HLA2_ERR_LAUNCH = -4       /* a kernel launch failed */
};

/* Human-readable text for a return code (static storage). */
const char *hla2_strerror(int code);

/* ABI version of this header (incremented on incompatible changes). */
int hla2_abi_version(void);

/*
 * Workspace needed by hla2_forward for this shape, in bytes (0 when the
 * sequence fits one segment).  Depends only on the arguments.  Returns 0 for
 * an invalid or unsupported shape as well; hla2_forward reports those.
 */
size_t hla2_forward_workspace_bytes(int B, int H, int n, int d, int dv, int chunk);

/*
 * Number of segments per (b, h) that hla2_forward uses for this shape (the
 * length of the scanned sequence of segment summaries), or a negative code.
 */
int hla2_forward_segments(int B, int H, int n, int d, int dv, int chunk);

/*
 * Masked second-order HLA forward pass: out_t = q_t^T (S_t C_t - G_t), or that
 * over q_t^T (S_t m_t - h_t) [SUM §1, output formula and normalisation],
 * computed chunk-parallel through segment summaries and an exclusive scan with
 * the semidirect-product combine [SUM §4, associative operators and scan
 * equivalence].
 *   q, k : [B, H, n, d]    element type `dtype`
 *   v    : [B, H, n, dv]   element type `dtype`
 *   out  : [B, H, n, dv]   element type `dtype` (written)
 *   decay: g in (0, 1]; 1 = no decay
 *   normalize: 0 -> out = num;  1 -> out = num / den
 *   chunk: tokens per chunk, one of 16, 32, 64, 128.  The result does not
 *          depend on it beyond rounding [SUM §4, scan equivalence].  The fp32
 *          path uses it as its tile; the bf16 path always walks 64-token chunks,
 *          so bf16 results are bitwise the same for every valid `chunk`.
 *   den_out: nullable [B, H, n] fp32; when given, den_t is written whatever
 *          `normalize` says
 *   workspace: device buffer of at least hla2_forward_workspace_bytes(...)
 *          bytes (may be NULL when that is 0); contents on entry are ignored
 * Supported: d, dv multiples of 16 in [16, 128]; n >= 1; B, H >= 1; one head's
 * rows in bytes, n * (max(d, dv) + 16) * 4, below 2^31 - 256 (they are addressed
 * with 32-bit offsets); B*H <= 2^24 and B*H*n <= 2^40; and B*H*segments*512 below
 * 2^32 (one workgroup per head and segment; larger grids give
 * HLA2_ERR_UNSUPPORTED).
 * Causality: for finite inputs, out_t and den_t are bitwise unchanged by any
 * change of tokens after t [SUM "Resultaten en claims"].  A NaN or Inf in a
 * later token can still reach earlier outputs, because the masked products
 * multiply it by zero (0 * Inf = NaN).
 */
int hla2_forward(const void *q, const void *k, const void *v, void *out,
                 int B, int H, int n, int d, int dv, float decay, int normalize, int chunk,
                 hla2_dtype_t dtype, float *den_out, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * One streaming step for N sequences x H heads, state updated in place
 * [SUM §1, state upkeep / output / normalisation; ABS: constant-size state].
 *   state: [N, H] blocks of fp32, each block laid out as
 *          S[d*d] | C[d*dv] | m[d] | G[d*dv] | h[d]   (row-major; see the
 *          definitions above), i.e. hla2_state_floats(d, dv) floats per block
 *   q, k : [N, H, d]   element type `dtype`
 *   v    : [N, H, dv]  element type `dtype`
 *   out  : [N, H, dv]  element type `dtype` (written)
 * Order inside the step: the cross summaries take the new key against the
 * OLD C and m, then S, C, m absorb the token, then the readout uses the new
 * state.  Supported: d, dv in {16, 32, 64, 128}; N*H below 2^24 (one 256-thread
 * workgroup per (sequence, head); larger counts give HLA2_ERR_UNSUPPORTED).
 */
int hla2_decode_step(float *state, const void *q, const void *k, const void *v, void *out,
                     int N, int H, int d, int dv, float decay, int normalize,
                     hla2_dtype_t dtype, hipStream_t stream);

/*
 * hla2_forward with an explicit segment count (a scheduling knob for tuning and
 * tests; the result does not depend on it beyond rounding).  segments = 0
 * picks the count hla2_forward uses; otherwise the requested count is clamped
 * to [1, min(number of chunks, 64)] and the chunks are split as evenly as
 * whole chunks allow.  The workspace must be sized with
 * hla2_forward_ex_workspace_bytes for the same `segments`.
 */
size_t hla2_forward_ex_workspace_bytes(int B, int H, int n, int d, int dv, int chunk, int segments);
int hla2_forward_ex_segments(int B, int H, int n, int d, int dv, int chunk, int segments);

/*
 * The segment plan of a bf16 hla2_forward_ex call with these arguments
 * [SUM §4: the sequence is cut into segments whose summaries are scanned].
 * Writes the number of segments per (b, h), the 64-token chunks of segment 0
 * and the chunks of every later segment (the last may hold fewer).  Returns 1
 * for a lead plan (segment 0 is walked for its outputs beside the summary
 * walks of segments 1 .. nseg-2 and leaves the incoming state of segment 1;
 * the scan starts there and the output walk covers segments 1 .. nseg-1),
 * 0 for a plain plan (summaries of segments 0 .. nseg-2, scan, output walk of
 * every segment), or a negative code (null pointer, segments < 0, unsupported
 * shape).  Host only: no device call.
 */
int hla2_forward_ex_plan(int B, int H, int n, int d, int dv, int chunk, int segments, int *nseg,
                         int *lead_chunks, int *seg_chunks);
int hla2_forward_ex(const void *q, const void *k, const void *v, void *out,
                    int B, int H, int n, int d, int dv, float decay, int normalize, int chunk,
                    hla2_dtype_t dtype, float *den_out, void *workspace, size_t workspace_bytes,
                    int segments, hipStream_t stream);

/*
 * hla2_forward_ex that also records HIP events on `stream` between its kernel
 * launches, so a caller can time each phase of the chunk-parallel pass
 * [SUM §4] on the stream the kernels run on.  `events` is NULL or an array of
 * four hipEvent_t (entries may be NULL; the caller creates and owns them):
 *   events[0] before the segment-summary kernel (with a lead plan, see
 *             hla2_forward_ex_plan: the launch that also walks segment 0's
 *             outputs),
 *   events[1] after it (before the segment scan),
 *   events[2] after the scan (before the chunk-output kernel),
 *   events[3] after the chunk-output kernel.
 * With one segment only the chunk-output kernel runs and events[0..2] are
 * recorded back to back; with a two-segment lead plan no scan runs and
 * events[1..2] are back to back.  Results are those of hla2_forward_ex.  A failed
 * hipEventRecord is reported as HLA2_ERR_LAUNCH.
 */
int hla2_forward_timed(const void *q, const void *k, const void *v, void *out,
                       int B, int H, int n, int d, int dv, float decay, int normalize, int chunk,
                       hla2_dtype_t dtype, float *den_out, void *workspace, size_t workspace_bytes,
                       int segments, hipEvent_t const *events, hipStream_t stream);

/* Floats per (sequence, head) state block: d*d + 2*d*dv + 2*d. */
long hla2_state_floats(int d, int dv);

/*
 * hla2_forward that also exports the state after the last token, in the
 * layout hla2_decode_step reads, so streaming decode continues where the
 * forward pass stopped [SUM §1, state upkeep; SUM §4: the inclusive total of
 * the scan is the state after the whole sequence].
 *   state_out: [B, H] blocks of hla2_state_floats(d, dv) fp32 (written),
 *          S[d*d] | C[d*dv] | m[d] | G[d*dv] | h[d] as for hla2_decode_step,
 *          equal (up to rounding) to the state the serial recurrence holds
 *          after token n-1.  Must not be NULL (HLA2_ERR_INVALID).
 *   workspace: at least hla2_forward_state_workspace_bytes(...) bytes for the
 *          same `segments`, 256-byte aligned; never 0 bytes, since every
 *          segment keeps its summary for the export.
 *   segments: as for hla2_forward_ex (0 = the automatic count).
 * All other arguments, outputs and errors are those of hla2_forward_ex.
 * Internally the summaries of every segment are
 * folded with the incoming prefix of the last one, and the tokens after the
 * last full chunk are absorbed one by one, in fp32.
 */
size_t hla2_forward_state_workspace_bytes(int B, int H, int n, int d, int dv, int chunk, int segments);
int hla2_forward_state(const void *q, const void *k, const void *v, void *out,
                       int B, int H, int n, int d, int dv, float decay, int normalize, int chunk,
                       hla2_dtype_t dtype, float *den_out, float *state_out, void *workspace,
                       size_t workspace_bytes, int segments, hipStream_t stream);

/*
 * Backward pass: the gradients of L = sum(dout * out) with respect to q, k and
 * v, for the forward of hla2_forward (same decay and normalisation).  The
 * pages run the chunk-parallel scan for training [SUM §4] but print no
 * gradient; it is the chain rule of the operation defined above:
 *   with M[t][j] = sum_{i<=j} g^{(t-i)+(t-j)} (q_t.k_i)(q_j.k_i) (j <= t),
 *   num = M V, den = M 1, and the upstream gradients g_num = dout, g_den = 0
 *   (normalize = 0) or g_num = dout / den, g_den = -(dout . out) / den
 *   (normalize = 1, using the forward's own out and den),
 *   dV = M^T g_num;  dq, dk through the scores q_t.k_i of both factors.
 * It runs as the adjoint of the chunked forward: a forward walk that stores
 * every chunk's incoming state, a reverse scan of adjoint segment summaries,
 * and a backward walk that writes the gradients.
 *   q, k : [B, H, n, d];  v, dout, out : [B, H, n, dv]   element type `dtype`
 *   den  : [B, H, n] fp32 (the forward's den_out)
 *   out, den: read only when normalize = 1 (may be NULL otherwise)
 *   grad_q, grad_k : [B, H, n, d];  grad_v : [B, H, n, dv]  (written, `dtype`)
 *   decay: g in (0, 1], a constant (no gradient is formed for it)
 *   workspace: device buffer of at least hla2_backward_workspace_bytes(...)
 *          bytes for the same arguments, 256-byte aligned; never 0 bytes
 *   segments: 0 picks the plan; otherwise as for hla2_forward_ex
 * Supported: as hla2_forward (bf16: d, dv multiples of 16 up to 128; fp32: up
 * to 64).  The chunking is internal (64 tokens for bf16 at d <= 64, else 32);
 * the results change only by rounding with it.  All tensor pointers 16-byte
 * aligned.  Errors as for hla2_forward; workspace problems give
 * HLA2_ERR_WORKSPACE, a missing out/den under normalize = 1 HLA2_ERR_INVALID.
 */
size_t hla2_backward_workspace_bytes(int B, int H, int n, int d, int dv, int normalize,
                                     hla2_dtype_t dtype, int segments);
int hla2_backward(const void *q, const void *k, const void *v, const void *out, const float *den,
                  const void *dout, void *grad_q, void *grad_k, void *grad_v,
                  int B, int H, int n, int d, int dv, float decay, int normalize,
                  hla2_dtype_t dtype, void *workspace, size_t workspace_bytes, int segments,
                  hipStream_t stream);

/*
 * AHLA, the asymmetric variant [SUM §2]: the operator Q (K^T Q)(K^T V), masked
 * like the second-order case (all indices at or before t):
 *   num_t = sum_{j<=t} sum_{i<=j} g^{t-i} (q_t.k_j)(q_j.k_i) v_i,   den_t the same with v_i -> 1,
 *   out_t = num_t, or num_t / den_t when normalize = 1 (IEEE division),
 * i.e. A_g A_g V with A_g = L o D_g o (Q K^T).  The pages name its summaries
 * P^KV, m^K, E, n but print no update; the reading used: P^KV and m^K are the
 * decayed key-value and key-mass prefixes and E_t = g E_{t-1} + k_t (q_t^T P^KV_t),
 * n_t likewise with m^K, so num_t = q_t^T E_t and den_t = q_t^T n_t.  Computed
 * chunk-parallel [SUM §4]: segment summaries (P^KV, m^K, E, n and the segment's
 * sum of k q^T), an exclusive scan with the combine
 *   E_AB = G_B E_A + E_B + G_B (sum_{j in B} k_j q_j^T) P^KV_A,
 * and the chunk outputs from each segment's incoming state.
 *   q, k : [B, H, n, d];  v, out : [B, H, n, dv]  element type `dtype`
 *   den_out: nullable [B, H, n] fp32 (written whatever `normalize` says)
 *   workspace: at least hla2_ahla_forward_workspace_bytes(...) bytes for the
 *          same shape, dtype and `segments`, 256-byte aligned (may be NULL when
 *          that is 0, i.e. one segment)
 *   segments: 0 picks the plan; otherwise as for hla2_forward_ex
 * Supported shapes, alignment and errors as for hla2_forward (the chunking is
 * internal: 64 tokens for bf16 at d <= 64, else 32).
 */
size_t hla2_ahla_forward_workspace_bytes(int B, int H, int n, int d, int dv, hla2_dtype_t dtype,
                                         int segments);
int hla2_ahla_forward(const void *q, const void *k, const void *v, void *out,
                      int B, int H, int n, int d, int dv, float decay, int normalize,
                      hla2_dtype_t dtype, float *den_out, void *workspace, size_t workspace_bytes,
                      int segments, hipStream_t stream);

/*
 * Third-order HLA [SUM §3]: the interaction A A^T A with A = Q K^T, masked so
 * that no index passes t:
 *   num_t = sum_{l<=t} sum_{j<=l} sum_{i<=l} g^{(t-j)+(t-l)+(t-i)} (q_t.k_j)(q_l.k_j)(q_l.k_i) v_i,
 *   den_t the same with v_i -> 1,  out_t = num_t or num_t / den_t,
 * i.e. (L o D_{g^2} o (A_g A^T)) (A_g V) with A = L o (Q K^T), A_g = D_g o A;
 * unmasked and undecayed it is q_t^T S^K S^Q P^KV.  Reading (the pages name the
 * moments and cross summaries but print no update): every moment decays by g
 * per token; the cross summaries are carried as one corrected accumulator
 * W_t = g^3 W_{t-1} + (S^K_t q_t)(P^KV_t^T q_t)^T.  Computed chunk-parallel
 * [SUM §4, third-order scans]: segment summaries with the segment-level maps
 * that fold an incoming (S^K, P^KV) into W, an exclusive scan, and the chunk
 * outputs from each segment's incoming state.
 *   Arguments, layouts, workspace and errors as for hla2_ahla_forward (with
 *   hla2_ho3_forward_workspace_bytes).  Supported: d <= 64 (the d x d state and
 *   maps are held on chip), dv as hla2_forward; fp32 up to 64.
 */
size_t hla2_ho3_forward_workspace_bytes(int B, int H, int n, int d, int dv, hla2_dtype_t dtype,
                                        int segments);
int hla2_ho3_forward(const void *q, const void *k, const void *v, void *out,
                     int B, int H, int n, int d, int dv, float decay, int normalize,
                     hla2_dtype_t dtype, float *den_out, void *workspace, size_t workspace_bytes,
                     int segments, hipStream_t stream);

/*
 * hla2_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * caller passes inputs and outputs only; the workspace hla2_forward would take
 * (segment summaries and prefixes) is a fixed device array the library holds,
 * HLA2_NOALLOC_SCRATCH_BYTES (96 MiB) on each device it runs on, from the
 * first call on that device until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments, layouts, results and errors as for hla2_forward, and
 *   HLA2_ERR_UNSUPPORTED when hla2_forward_workspace_bytes(...) for the shape
 *   exceeds HLA2_NOALLOC_SCRATCH_BYTES (96 MiB holds the workspace of, e.g.,
 *   8 x 16 heads of 8192 tokens at d = 64, dv = 128, or 16 heads of 65536
 *   tokens at d = dv = 128); HLA2_ERR_LAUNCH when the array's device address
 *   cannot be obtained.
 *   The array's contents on entry are ignored (every byte the call reads it
 *   writes first), so nothing has to be cleared between calls.
 *   Every call on one device shares that device's array: calls that overlap on
 *   one device (different streams, threads or processes' graphs without
 *   ordering) race on it and give wrong results.  Order them (one stream, or
 *   events).
 */
#define HLA2_NOALLOC_SCRATCH_BYTES (96u << 20)
int hla2_forward_noalloc(const void *q, const void *k, const void *v, void *out,
                         int B, int H, int n, int d, int dv, float decay, int normalize, int chunk,
                         hla2_dtype_t dtype, float *den_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HLA2_H_ */
