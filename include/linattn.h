/*
 * linattn.h -- C ABI of the causal linear-attention library for AMD Instinct
 * MI355X (gfx950).  Plain C: pointers, sizes and integer codes only.
 *
 * The method.  Attention is the dot product of kernel feature maps phi
 * ("Transformers are RNNs: Fast Autoregressive Transformers with Linear
 * Attention", abstract).  For causal inputs the output at position i is
 *     y_i = phi(q_i) (sum_{j<=i} phi(k_j)^T v_j) / phi(q_i) (sum_{j<=i} phi(k_j)^T)
 * and the sums are carried as a value state S (D x d_v) and a key state z (D):
 *     S_i = S_{i-1} + phi(k_i)^T v_i,  z_i = z_{i-1} + phi(k_i)^T,
 *     y_i = phi(q_i) S_i / phi(q_i) z_i
 * ("Simple linear attention language models balance the recall-throughput
 * tradeoff", Knowl 3, both equations).
 *
 * Feature maps (linattn_map_t):
 *   LINATTN_MAP_ELU1    phi(x) = elu(x) + 1 elementwise, alpha = 1; D = d_k.
 *   LINATTN_MAP_TAYLOR2 phi(x) = [1, x, vec(x (x) x)/sqrt(2)], row-major vec
 *                       (feature 1 + d_k + a*d_k + b is x_a x_b / sqrt 2);
 *                       D = 1 + d_k + d_k^2, so phi(q).phi(k) = 1 + q.k +
 *                       (q.k)^2/2 (same page, Knowl 3).
 *   LINATTN_MAP_TAYLOR2_SYM  the same kernel with each unordered pair of
 *                       coordinates counted once: phi(x) = [1, x, w_ab x_a x_b
 *                       for a <= b], pairs in row-major upper-triangular
 *                       order (feature 1 + d_k + a*d_k - a(a-1)/2 + (b-a)),
 *                       w_aa = 1/sqrt(2), w_ab = 1 for a < b;
 *                       D = 1 + d_k + d_k(d_k+1)/2 = 153 at d_k = 16, the
 *                       state size of the generation-state accounting (same
 *                       page, Knowl 7).  phi(q).phi(k) equals TAYLOR2's.
 *                       Its state relates to TAYLOR2's by
 *                       S_sym[{a,b}] = (S[a,b] + S[b,a]) / sqrt(2), a < b, and
 *                       S_sym[{a,a}] = S[a,a].
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library allocates and frees nothing and keeps no global state, except
 *     the fixed device array of linattn_prefill_noalloc.
 *   - Tensors are contiguous, row-major, and their base address is 16-byte
 *     aligned.  q, k, v, y share one element type (linattn_dtype_t); the
 *     states S, z are always float32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return; they never synchronise the host.
 *   - Arguments are validated on the host before anything is launched.  On
 *     a non-zero status nothing has been enqueued and nothing written.  A
 *     launch failure reported by the HIP runtime returns LINATTN_ERR_HIP.
 *   - Outputs must not overlap inputs, except where a call says otherwise.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics).
 *   - Supported shapes (anything else returns LINATTN_ERR_UNSUPPORTED):
 *       ELU1:    d_k == d_v in {16, 32, 64}
 *       TAYLOR2: d_k == 16, d_v in {16, 32, 64}   (D = 273)
 *       TAYLOR2_SYM: d_k == 16, d_v in {16, 32, 64}   (D = 153)
 *     for both dtypes, any B, H >= 1 and any N >= 1 (ragged tails are
 *     masked inside the kernels).
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum linattn_status {
  LINATTN_OK = 0,
  LINATTN_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, size <= 0, misaligned */
  LINATTN_ERR_UNSUPPORTED = 2,      /* valid but not built: map/dtype/d_k/d_v */
  LINATTN_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  LINATTN_ERR_HIP = 4,              /* the HIP runtime rejected a launch */
  LINATTN_ERR_SCRATCH = 5           /* linattn_prefill_noalloc: the call needs
                                       more than its fixed scratch array */
} linattn_status_t;

/* Bytes of the fixed device array of linattn_prefill_noalloc (per device). */
#define LINATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum linattn_map {
  LINATTN_MAP_ELU1 = 0,
  LINATTN_MAP_TAYLOR2 = 1,
  LINATTN_MAP_TAYLOR2_SYM = 2
} linattn_map_t;

typedef enum linattn_dtype {
  LINATTN_DTYPE_F32 = 0,
  LINATTN_DTYPE_BF16 = 1
} linattn_dtype_t;

/* Every entry point takes its map and dtype codes (the values above) as
   plain int, so that any value a caller passes reaches validation and an
   unknown code returns LINATTN_ERR_INVALID_ARGUMENT rather than being an
   out-of-range enum inside the library. */

/* Static text for a status code (never NULL). */
const char* linattn_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int linattn_version(void);

/* Feature dimension D of a map: ELU1 -> d_k; TAYLOR2 -> 1 + d_k + d_k^2;
   TAYLOR2_SYM -> 1 + d_k + d_k(d_k+1)/2.
   Returns -1 for an unknown map or d_k <= 0. */
int64_t linattn_feature_dim(int map, int64_t d_k);

/* 1 if (map, dtype, d_k, d_v) is one of the built kernel shapes, else 0. */
int linattn_supported(int map, int dtype, int64_t d_k, int64_t d_v);

/*
 * phi(x) for every row of x, written to HBM as float32.
 *   x   [rows, d_k] of `dtype`;  phi [rows, D] float32, D = feature_dim.
 * Feature maps as defined above ("Simple linear attention ...", Knowl 3).
 * This export exists for tests and inspection; the attention calls never
 * materialise phi in HBM (same page, Knowl 5, last paragraph).
 * Supported: the d_k values listed above.  rows == 0 is a no-op.
 */
linattn_status_t linattn_feature_map(int map, int dtype, const void* x,
                                     int64_t rows, int64_t d_k, float* phi,
                                     void* stream);

/*
 * Bytes of device workspace linattn_prefill and linattn_prefill_gated need
 * for this shape and segment length (0 = the library's choice).  May be 0.
 * Returns (size_t)-1 for invalid or unsupported arguments.
 */
size_t linattn_prefill_workspace_bytes(int map, int dtype, int64_t B,
                                       int64_t H, int64_t N, int64_t d_k,
                                       int64_t d_v, int64_t seg_len);

/*
 * Causal prefill: every output y_i of the causal equation above for all
 * B*H sequences of length N, and optionally the final state for later
 * generation ("Simple linear attention ...", Knowl 5, first paragraph:
 * prefill takes q, k, v for B, H, N, d and D, and may write the final
 * states).
 *   q  [B, H, N, d_k]   k [B, H, N, d_k]   v [B, H, N, d_v]   (dtype)
 *   y  [B, H, N, d_v]   (dtype; bf16 results are rounded to nearest even)
 *   S_in, z_in  [B, H, D, d_v], [B, H, D] float32: the state before token 1,
 *               or both NULL for the zero state (the sums of the causal
 *               equation then start at j = 1).
 *   S_out, z_out [B, H, D, d_v], [B, H, D] float32: the state after token N,
 *               or both NULL.  S_out may be the same pointer as S_in and
 *               z_out the same as z_in (in-place continuation); any other
 *               overlap is an error.  In place, a plan of several segments
 *               per head always forms the segment prefixes in a separate
 *               launch that reads S_in, z_in before any output workgroup
 *               runs, so no workgroup can read a state already overwritten.
 *   seg_len     tokens per workgroup segment along N: 0 = library choice,
 *               else a positive multiple of 64.  Results agree for every
 *               choice to rounding; each choice is deterministic.
 *   workspace   device scratch of at least
 *               linattn_prefill_workspace_bytes(..., seg_len) bytes (may be
 *               NULL when that is 0).  Its contents on entry do not matter;
 *               on return they are unspecified.  Two calls in flight at once
 *               must not share a workspace.
 * Internally the state is accumulated in float32; bf16 inputs feed bf16
 * MFMA products with float32 accumulation.
 */
linattn_status_t linattn_prefill(int map, int dtype, int64_t B, int64_t H,
                                 int64_t N, int64_t d_k, int64_t d_v,
                                 const void* q, const void* k, const void* v,
                                 void* y, const float* S_in,
                                 const float* z_in, float* S_out, float* z_out,
                                 int64_t seg_len, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * linattn_prefill without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Every argument means what it means for
 * linattn_prefill; the segment part sums go to a fixed device array that
 * the library holds on each device it runs on (LINATTN_NOALLOC_SCRATCH_BYTES,
 * 64 MiB, kept until the process ends).  The call allocates nothing and
 * frees nothing; on its first use on a device it looks up that array's
 * device address (the device current at the call, which must be the
 * stream's device).
 *   Returns LINATTN_ERR_SCRATCH, before anything is launched, when
 *   linattn_prefill_workspace_bytes(map, dtype, B, H, N, d_k, d_v, seg_len)
 *   exceeds LINATTN_NOALLOC_SCRATCH_BYTES (a Taylor part sum at d_v = 64
 *   takes 51,200 bytes per head and part, so B=8 H=16 N=2048 needs 26 MB;
 *   ELU1 at d = 64 takes 20,480); other errors as linattn_prefill.
 *   All calls on one device share its array: two calls that may run at the
 *   same time on one device (different streams, no ordering between them)
 *   race and give wrong results.  Calls ordered on one stream are safe;
 *   what a call leaves in the array does not matter to the next one.
 */
linattn_status_t linattn_prefill_noalloc(int map, int dtype, int64_t B, int64_t H,
                                         int64_t N, int64_t d_k, int64_t d_v,
                                         const void* q, const void* k, const void* v,
                                         void* y, const float* S_in, const float* z_in,
                                         float* S_out, float* z_out, int64_t seg_len,
                                         void* stream);

/*
 * Gated (scalar-decay) causal prefill.  The state is scaled by a per-token
 * coefficient a_t before the token is added (the gated linear recurrences
 * of the Hacker News discussion of "Transformers are RNNs", "In the
 * conversation": a forget factor that is a scalar times the identity, which
 * the same discussion relates to state-space layers with scalar
 * transitions through compounded coefficients a_1 ... a_t):
 *     S_t = a_t S_{t-1} + phi(k_t)^T v_t,   z_t = a_t z_{t-1} + phi(k_t)^T,
 *     y_t = phi(q_t) S_t / phi(q_t) z_t   (normalize = 1)
 *     y_t = phi(q_t) S_t                  (normalize = 0).
 * Unrolled, token j counts at position i with weight a_{j+1} ... a_i.
 *   gate  [B, H, N] float32 device pointer, 4-byte aligned: a_t, meant to lie
 *         in [0, 1] (a = 1 everywhere is the plain prefill; a = 0 drops all
 *         earlier tokens and the initial state).  Coefficients below 2^-64
 *         are taken as exactly 0 (a change below 2^-64 relative).  Values
 *         outside [0, 1] are not checked: they are used as given (> 1
 *         grows the state), and NaN or negative values give unspecified
 *         outputs.  Never written; must not overlap y, S_out or z_out.
 *   normalize  1 or 0 as above; anything else is an invalid argument.
 * Every other argument, the workspace and the supported shapes are those of
 * linattn_prefill; S_in (if given) is decayed by a_1 like any earlier state.
 * The weights are formed in float32 as 2^(G_i - G_j) from running sums G of
 * log2 a_t within each 64-token chunk, so the relative error of a weight
 * grows with the magnitude of those sums (about 1e-5 for |G| <= 100).
 */
linattn_status_t linattn_prefill_gated(int map, int dtype, int64_t B, int64_t H,
                                       int64_t N, int64_t d_k, int64_t d_v,
                                       const void* q, const void* k, const void* v,
                                       const float* gate, int normalize, void* y,
                                       const float* S_in, const float* z_in,
                                       float* S_out, float* z_out, int64_t seg_len,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * One generation step for all B*H sequences: update the state with the new
 * token, then read it ("Simple linear attention ...", Knowl 3 recurrent
 * equations; Knowl 5, second paragraph):
 *   S += phi(k)^T v;  z += phi(k)^T;  y = phi(q) S / phi(q) z.
 *   q, k [B, H, d_k]   v [B, H, d_v]   y [B, H, d_v]   (dtype)
 *   S [B, H, D, d_v], z [B, H, D] float32, read and written in place.
 * All arithmetic is float32 (inputs are widened); y is rounded to dtype.
 * y must not overlap S or z.  A zero state is valid input only if the step's
 * own token makes the denominator positive (it always does: phi(k) > 0 for
 * ELU1 and phi(q).phi(k) >= 1/2 for both Taylor maps).
 */
linattn_status_t linattn_decode_step(int map, int dtype, int64_t B, int64_t H,
                                     int64_t d_k, int64_t d_v, const void* q,
                                     const void* k, const void* v, float* S,
                                     float* z, void* y, void* stream);

/*
 * One gated generation step (the recurrence of linattn_prefill_gated):
 *   S = a S + phi(k)^T v;  z = a z + phi(k)^T;  y = phi(q) S [/ phi(q) z].
 *   gate [B, H] float32 device pointer, 4-byte aligned: this step's a per
 *        sequence and head, used exactly as given (no 2^-64 cut-off here).
 *   normalize 1 (ratio) or 0 (numerator only).
 * Otherwise as linattn_decode_step; gate must not overlap y, S or z.
 */
linattn_status_t linattn_decode_step_gated(int map, int dtype, int64_t B, int64_t H,
                                           int64_t d_k, int64_t d_v, const void* q,
                                           const void* k, const void* v,
                                           const float* gate, int normalize, float* S,
                                           float* z, void* y, void* stream);

/*
 * Sliding-window softmax attention, prefill ("Simple linear attention ...",
 * Knowl 4: query i attends only to keys max(1, i-w+1) .. i; the BASED
 * model pairs it with the Taylor linear attention).  For every position i
 * (0-based) of every sequence and head:
 *     p_ij = softmax over j in [max(0, i-w+1), i] of scale * q_i . k_j,
 *     y_i  = sum_j p_ij v_j.
 *   q, k, v, y  [B, H, N, d] of `dtype` (d_k = d_v = d); d in {32, 64, 128}.
 *   window      w >= 1 (w >= N is causal softmax attention).
 *   scale       any finite float, or NaN for the usual 1/sqrt(d).
 *   k_cache, v_cache  [B, H, w, d] of `dtype`, or both NULL: when given,
 *               they receive the ring cache that linattn_swa_decode_step
 *               continues from -- token t (t >= N - w) in slot t mod w,
 *               zeros in slots no token has reached (N < w).
 * Scores, the running maximum and the sums are float32; bf16 inputs feed
 * bf16 MFMA products, and the softmax weights enter the value product as
 * bf16.  y is rounded to dtype.  One sequence's rows must stay below 2 GiB.
 * No workspace; outputs must not overlap inputs or each other.
 */
linattn_status_t linattn_swa_prefill(int dtype, int64_t B, int64_t H, int64_t N,
                                     int64_t d, int64_t window, float scale,
                                     const void* q, const void* k, const void* v,
                                     void* y, void* k_cache, void* v_cache,
                                     void* stream);

/*
 * Sliding-window generation step (same page, Knowl 4: a w-token key-value
 * cache; Knowl 5: the generation kernel fuses the query-key product, the
 * softmax and the value product).  For every sequence b and head h at the
 * 0-based position p = pos[b]: write k, v into slot p mod w of the caches,
 * then attend over the min(p + 1, w) tokens p - w + 1 .. p held there.
 *   q, k, v, y  [B, H, d] of `dtype`;  d in {32, 64, 128}.
 *   pos         [B] int64 device array, 8-byte aligned, read only (the
 *               caller advances it); a negative entry makes that sequence's
 *               y NaN and leaves its cache unchanged.
 *   k_cache, v_cache  [B, H, w, d] of `dtype`, updated in place; slots not
 *               yet reached are never read.
 *   window      1 <= w <= 4096 (else LINATTN_ERR_UNSUPPORTED).
 *   scale       as for linattn_swa_prefill (NaN: 1/sqrt(d)).
 * All arithmetic is float32; y is rounded to dtype.
 */
linattn_status_t linattn_swa_decode_step(int dtype, int64_t B, int64_t H, int64_t d,
                                         int64_t window, float scale, const void* q,
                                         const void* k, const void* v, const int64_t* pos,
                                         void* k_cache, void* v_cache, void* y,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
