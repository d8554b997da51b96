/*
 * seed.h -- C ABI of the MI355X (gfx950) shallow recurrent-state engine.
 *
 * A linear-attention / state-space head keeps a d_k x d_v recurrent state S.
 * SEED stores it as a sink along a fixed per-head direction plus rank-R
 * factors,  S = a vbar^T + U V^T  (SEED summary on picx.dev, "SEED
 * Architecture"; SEED figures and tables on thelatestinai.com, Fig. 1 (b)).
 * Each decode step reads the state out and applies the head's gated update
 * exactly by rescaling a, decaying U and appending one column to U and V
 * (picx.dev summary, "Exact Update (Lemma 2)"); every W steps the factors
 * are compressed back to rank R (Fig. 1 (b) caption).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  Base pointers must be 16-byte
 *    aligned.  Arrays are dense, row-major, in the layouts given below.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; nothing synchronises.  Calls on the
 *    same state must be serialised by the caller (same stream or events).
 *  - Every call validates its arguments on the host BEFORE touching the HIP
 *    runtime and returns a seed_status.  Nothing aborts, throws or prints.
 *    On failure nothing was launched and seed_last_error() (thread-local)
 *    describes the problem.  A kernel fault surfaces at the caller's next
 *    synchronisation, not here.
 *  - NaN / Inf inputs are not checked; they propagate into the outputs.
 *  - Supported head shapes (d_k, d_v): (128,128), (128,64), (64,64).
 *    Factor capacity cap = R + W <= 96 columns.  Larger or other shapes
 *    return SEED_E_UNSUPPORTED.
 *
 * Layouts, for `batch` requests of `heads` heads (unit index b*heads + h):
 *   a    float [batch][heads][d_k]          sink coefficients
 *   U    float [batch][heads][cap][d_k]     factor columns; column j of U is
 *                                           the contiguous U[b][h][j][:]
 *   V    float [batch][heads][cap][d_v]     factor columns, same scheme
 *   vbar float [heads][d_v]                 per-head direction, shared by
 *                                           all requests; any nonzero vector
 *   S    float [batch][heads][d_k][d_v]     dense state (row i = key i)
 *   q, k       [batch][heads][d_k]          fp32 or bf16 (see in_dtype)
 *   v          [batch][heads][d_v]          fp32 or bf16
 *   g    float [batch][heads]               decay (Gated DeltaNet, Mamba-2)
 *        float [batch][heads][d_k]          decay per key channel (KDA)
 *   beta float [batch][heads]               write strength (NULL for Mamba-2)
 *   o    float [batch][heads][d_v]          read-out (must not alias inputs)
 *
 * The factor columns form a ring of fixed capacity: a step writes column r
 * (never moves data), compression rewrites columns 0..R-1.  The caller keeps
 * r, the number of columns held, which is the same for the whole batch.
 */
#ifndef SEED_H
#define SEED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SEED_OK = 0,
  SEED_E_ARG = 1,          /* NULL or misaligned pointer, unknown enum value   */
  SEED_E_SHAPE = 2,        /* sizes that contradict each other or are <= 0     */
  SEED_E_UNSUPPORTED = 3,  /* valid, but outside the shapes this build covers  */
  SEED_E_FULL = 4,         /* decode step asked for with r == cap: compress first */
  SEED_E_DEVICE = 5        /* the HIP runtime refused the launch               */
} seed_status;

typedef enum {
  SEED_RULE_GDN = 0,    /* Gated DeltaNet:        S' = g (I - beta k k^T) S + beta k v^T      */
  SEED_RULE_KDA = 1,    /* Kimi Delta Attention:  S' = (I - beta k k^T) Diag(g) S + beta k v^T */
  SEED_RULE_MAMBA2 = 2  /* Mamba-2 (d_k = state dim, d_v = head dim):  S' = g S + k v^T    */
} seed_rule;

/* Storage types.  q, k, v: SEED_F32 or SEED_BF16.  Kept factors of the
 * 16-bit form (seed_decode_step_h16 and after): SEED_BF16 or SEED_F16. */
typedef enum { SEED_F32 = 0, SEED_BF16 = 1, SEED_F16 = 2 } seed_dtype;

typedef enum {
  SEED_ROUND_NEAREST = 0,    /* IEEE round to nearest, ties to even               */
  SEED_ROUND_STOCHASTIC = 1  /* up with probability (|x| - lo)/(hi - lo), Philox words */
} seed_rounding;

/*
 * seed_decode_step -- one decode step of every (request, head) unit.
 *
 * Defined by Lemma 2 (picx.dev summary, "Exact Update (Lemma 2)"), with
 * omega = v.vbar/|vbar|^2 and eps = v - omega vbar:
 *   Gated DeltaNet:  a <- g a + beta (omega - g k.a) k
 *                    U <- [g U, k],  V <- [V, beta (eps - V (g U)^T k)]
 *   Kimi Delta Attention: the same with Diag(g) for the scalar g.
 *   Mamba-2:         a <- g a + omega k,  U <- [g U, k],  V <- [V, eps]
 * then the read-out of the updated state, o = vbar (a.q) + V (U^T q)
 * (SEED figures and tables, Table 1: the factors give the read-out and the
 * exact update).  U is decayed in place.  `r` is the number of columns held
 * on entry (0 <= r < cap); on return r + 1 columns are held.
 * Returns SEED_E_FULL if r == cap.  `beta` must be NULL for Mamba-2 and
 * non-NULL otherwise.  All factor and output arithmetic is fp32; bf16
 * inputs are widened exactly.
 */
seed_status seed_decode_step(int rule, int batch, int heads, int d_k, int d_v, int cap, int r,
                             float *a, float *U, float *V, const float *vbar,
                             const void *q, const void *k, const void *v, int in_dtype,
                             const float *g, const float *beta, float *o, void *stream);

/*
 * seed_compress -- compress the factors of every unit from r to R columns.
 *
 * Replaces the content U V^T by its best rank-R approximation (truncated
 * SVD) and leaves the sink coefficient a untouched: every W steps the
 * factors are compressed back to rank R (SEED figures and tables, Fig. 1 (b)
 * caption); the sink is preserved exactly (sungsoo.github.io summary,
 * method list, "Decode").  On return columns 0..R-1 hold U' with orthonormal
 * columns and V' = M^T U' (M = the old U V^T), so U' V'^T is the rank-R
 * truncation; the caller sets r = R.  If r <= R nothing is launched and
 * SEED_OK is returned.  Computed in fp32 in one workgroup per unit.
 */
seed_status seed_compress(int batch, int heads, int d_k, int d_v, int cap, int r, int R,
                          float *U, float *V, void *stream);

/*
 * seed_decode_step_lazy -- the step of seed_decode_step with the decay of U
 * kept as a running product instead of being applied in place.
 *
 *   gam  float [batch][heads][d_k]   decay product per key channel (KDA)
 *        float [batch][heads]        one decay product per unit (GDN, Mamba-2)
 *
 * The stored columns are U~ with U = Diag(gam) U~ (GDN and Mamba-2:
 * U = gam U~).  A step sets gam <- g gam (per channel for KDA), appends
 * U~_r = k / gam and leaves every other column of U~ as it is: only the
 * write-back of the decayed U disappears.  The update and read-out are
 * those of seed_decode_step (Lemma 2, picx.dev summary, "Exact Update
 * (Lemma 2)"; the caption of Table 2 of the SEED figures and tables has U
 * rescaled at every step, which gam does implicitly), so a, V and o agree
 * with it up to fp32 rounding.  A state from seed_state_from_dense or
 * seed_compress is in this form with gam = 1; compress with
 * seed_compress_lazy, which resets gam to 1.  gam is read and written.
 * The product must stay a normal fp32 number, so a step whose product for
 * a key channel falls below 2^-64 applies it to that row of every held
 * column (the in-place decay, for that channel) and restarts it at 1; the
 * represented state is the same, and gates of any size (down to 0) are
 * valid.
 */
seed_status seed_decode_step_lazy(int rule, int batch, int heads, int d_k, int d_v, int cap, int r,
                                  float *a, float *U, float *V, float *gam, const float *vbar,
                                  const void *q, const void *k, const void *v, int in_dtype,
                                  const float *g, const float *beta, float *o, void *stream);

/*
 * seed_compress_lazy -- seed_compress for the form of seed_decode_step_lazy:
 * the content Diag(gam) U~ V^T is replaced by its rank-R truncation,
 * stored as U' (orthonormal, true scale) and V' in columns 0..R-1, and gam
 * is set to 1.  `rule` selects the layout of gam (per key channel for
 * KDA).  If r <= R nothing is launched and gam is left as it is.
 */
seed_status seed_compress_lazy(int rule, int batch, int heads, int d_k, int d_v, int cap, int r,
                               int R, float *U, float *V, float *gam, void *stream);

/*
 * The 16-bit form: factors kept in fp16 or bf16 (SEED figures and tables,
 * Table 4 and its caption: 16-bit storage composes with the shallow state;
 * Table 9 and its caption: the factors rounded to nearest or stochastically
 * at every compression).  Read here as: the R columns a compression writes
 * are rounded once and kept as 16-bit patterns; the columns appended until
 * the next compression are fp32; nothing else is rounded.  The decay of U is
 * lazy, as in seed_decode_step_lazy.
 *
 *   Uk  uint16 [batch][heads][R][d_k]  kept columns of U~ (bf16 or fp16 patterns)
 *   Vk  uint16 [batch][heads][R][d_v]  kept columns of V
 *   Uw  float  [batch][heads][W][d_k]  columns of U~ appended since the last compression
 *   Vw  float  [batch][heads][W][d_v]  columns of V appended since the last compression
 *   gam float  as for seed_decode_step_lazy
 *
 * The state holds r columns, R <= r <= R + W: column j < R is column j of
 * Uk / Vk, column j >= R is column j - R of Uw / Vw.  Right after a
 * compression r = R.  Built for R = 16 or 32 (other R: SEED_E_UNSUPPORTED)
 * and R + W <= 96.
 *
 * Stochastic rounding: element f of a unit's block -- U column c row i at
 * f = c d_k + i, V column c row i at f = R d_k + c d_v + i -- takes the word
 * w = word (f mod 4) of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
 * at counter (f / 4, unit, epoch, 0) and key (seed mod 2^32, seed / 2^32),
 * and rounds its magnitude up iff (|x| - lo)/(hi - lo) > (w >> 8) 2^-24, with
 * lo <= |x| < hi the neighbouring 16-bit magnitudes.  Pass a new epoch (for
 * example the number of compressions so far) to every call.  fp16 overflows
 * to infinity from 2^16 (stochastic) or 65520 (nearest) up.
 */

/*
 * seed_decode_step_h16 -- seed_decode_step_lazy on the 16-bit form: reads
 * the kept columns (widened exactly) and the r - R appended ones, appends
 * column r (to Uw / Vw at index r - R, fp32) and writes a, gam and o as the
 * lazy step does.  Vk is only read; Uk is written only where a decay product
 * below 2^-64 is folded into a key row (seed_decode_step_lazy), that row of
 * every kept column then rounded to nearest -- entries at most 2^-64 of
 * their stored size, which no other term of the state can resolve.
 * Returns SEED_E_FULL if r == R + W.  store_dtype: SEED_BF16 or SEED_F16.
 */
seed_status seed_decode_step_h16(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                 int r, float *a, void *Uk, const void *Vk, float *Uw,
                                 float *Vw, float *gam, const float *vbar, const void *q,
                                 const void *k, const void *v, int in_dtype, int store_dtype,
                                 const float *g, const float *beta, float *o, void *stream);

/*
 * seed_compress_h16 -- compression of the 16-bit form: the content
 * Diag(gam) U~ V^T of the r columns is replaced by its rank-R truncation
 * (as seed_compress_lazy), computed in fp32, and U' (orthonormal) and V' are
 * rounded into Uk / Vk with the given rounding; gam is set to 1 and the
 * caller sets r = R.  If r <= R nothing is launched.  Uw / Vw are only
 * read.  `rule` selects the layout of gam.
 */
seed_status seed_compress_h16(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                              int r, void *Uk, void *Vk, float *Uw, float *Vw, float *gam,
                              int store_dtype, int rounding, uint64_t seed, uint32_t epoch,
                              void *stream);

/*
 * seed_round_factors -- round fp32 rank-R factors U [batch][heads][R][d_k],
 * V [batch][heads][R][d_v] (for example the output of seed_state_from_dense
 * with cap = R) into the kept columns Uk, Vk of the 16-bit form, with the
 * element numbering and words of seed_compress_h16.  U and V are only read;
 * they must not overlap Uk, Vk.  Requires 0 < R <= 96.
 */
seed_status seed_round_factors(int batch, int heads, int d_k, int d_v, int R, const float *U,
                               const float *V, void *Uk, void *Vk, int store_dtype, int rounding,
                               uint64_t seed, uint32_t epoch, void *stream);

/*
 * Per-request schedules.  Requests start at different times, so each has
 * its own column count and its own compression step (the pages compress
 * every W steps: SEED figures and tables, Fig. 1 (b) caption).  Request b
 * has taken A = t - t_start[b] steps at step t (it is idle, and its
 * read-out zero, while A < 0).  When its window reaches W columns (after
 * its step number k W) its content [R kept | W window] is compressed while
 * it keeps stepping; D steps later (A = k W + D) the truncation, decayed
 * by those steps' gates, replaces the compressed columns and the D columns
 * appended since are kept.  D = 0 compresses before the next step: the
 * aligned reading per request.  The decay of U is lazy as in
 * seed_decode_step_lazy.
 *
 *   t_start  int   [batch]                    step at which request b starts
 *   KU       float [2][batch][heads][R][d_k]  kept columns of U~, two buffers
 *   KV       float [2][batch][heads][R][d_v]  kept columns of V
 *   Uw       float [batch][heads][W + D][d_k] window ring: column number j
 *   Vw       float [batch][heads][W + D][d_v]   of a request in slot j mod (W + D)
 *   gam      float as for seed_decode_step_lazy (the running decay product)
 *   gam_snap float same shape: the product at the latest snapshot
 * With c = (A < W + D ? 0 : (A - D) / W) merges done, a request's kept
 * columns are buffer c & 1 and its window the column numbers c W .. A - 1;
 * it holds R + A - c W columns.  A state converted by seed_state_from_dense
 * (cap = R) goes into buffer 0 with gam = 1 and an empty window.
 * Built for R = 16 or 32, 0 <= D < W and R + W + D <= 96.
 *
 * seed_decode_step_sched -- step t of every request (Lemma 2 as in
 * seed_decode_step_lazy); at A = k W + D it first folds gam into every held
 * column and restarts gam at 1; at (A + 1) mod W = 0 it also stores the new
 * gam in gam_snap.  A product below 2^-64 is folded in as in
 * seed_decode_step_lazy, except in the D steps between a snapshot and its
 * merge (k W <= A < k W + D), where the snapshot's compression may still
 * read the held columns: there a product below 2^-110 makes the request's
 * gam NaN, so its read-outs are NaN from then on (D = 0 has no such steps).
 *
 * seed_compress_sched -- compress the units units[0 .. n_units) whose
 * request, at A = t_snap - t_start[b] steps, has taken its snapshot number
 * k = A / W >= 1 and not yet reached its merge: A - k W < D (A = k W when
 * D = 0).  Other listed units are left alone; entries outside the batch
 * are skipped.  Each is the rank-R truncation of snapshot k into kept
 * buffer k & 1, scaled by 1 / gam_snap.  Call it with t_snap = t + 1 after
 * step t, on any stream ordered after that step; the merge step of every
 * unit it compresses must be ordered after it.  So one call can serve the
 * requests whose snapshots fell in the last few steps, which amortises the
 * launch over more units.  Compressing a snapshot again before its merge
 * writes the same result.  Reads Uw, Vw and the old kept buffer; writes
 * only the new kept buffer.
 */
seed_status seed_decode_step_sched(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                   int D, int t, const int *t_start, float *a, float *KU,
                                   float *KV, float *Uw, float *Vw, float *gam, float *gam_snap,
                                   const float *vbar, const void *q, const void *k,
                                   const void *v, int in_dtype, const float *g, const float *beta,
                                   float *o, void *stream);

seed_status seed_compress_sched(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                int D, int t_snap, const int *t_start, int n_units,
                                const int *units, float *KU, float *KV, const float *Uw,
                                const float *Vw, const float *gam_snap, void *stream);

/*
 * Handoff of shallow-form states (prefill -> decode).  At the end of the
 * prefill a state is compressed to the sink plus rank-R factors (SEED
 * figures and tables, Fig. 1 (a) caption, Table 1), 4 [d_k + (d_k + d_v) R]
 * bytes per head in fp32 (Table 17 at w = 0; half the factor bytes in the
 * 16-bit form).  Packed layout: the selected requests one after another,
 * each with its heads in order, each head
 *     a [d_k] fp32 | U columns 0..R-1 [R][d_k] | V columns 0..R-1 [R][d_v]
 * with the factors in the state's storage type, seed_handoff_head_bytes()
 * bytes per head.  store_dtype SEED_F32: U, V are the fp32 column rings
 * [batch][heads][cap][d]; SEED_BF16 / SEED_F16: the kept arrays Uk, Vk of
 * the 16-bit form, [batch][heads][R][d] (pass cap = R).  The state must be
 * right after a compression or conversion (r = R; a lazy form's gam is 1
 * then), so that columns 0..R-1 are the whole state at true scale.
 * sel / slot: device int arrays of n_sel request indices; an index outside
 * [0, batch) selects nothing (its part of the buffer, or its slot, is left
 * as it was).  buf: device memory of n_sel * heads * head bytes, 16-byte
 * aligned, not overlapping the state.
 */

/* Bytes of one packed head (0 for an unsupported shape or dtype). */
size_t seed_handoff_head_bytes(int d_k, int d_v, int R, int store_dtype);

/* seed_pack_states -- copy requests sel[0..n_sel) of a state into buf. */
seed_status seed_pack_states(int batch, int heads, int d_k, int d_v, int cap, int R,
                             int store_dtype, int n_sel, const int *sel, const float *a,
                             const void *U, const void *V, void *buf, void *stream);

/* seed_unpack_states -- write the n_sel packed requests of buf into batch
 * slots slot[0..n_sel): a and columns 0..R-1 of U and V. */
seed_status seed_unpack_states(int batch, int heads, int d_k, int d_v, int cap, int R,
                               int store_dtype, int n_sel, const int *slot, const void *buf,
                               float *a, void *U, void *V, void *stream);

/*
 * seed_join_states -- requests that arrive while a batch is mid-window join
 * its compression phase.  For every slot[i] (an index outside [0, batch)
 * selects nothing): a and columns 0..R-1 of U and V are written from buf
 * (the layout of seed_pack_states with fp32 factors, e.g. a request packed
 * right after its end-of-prefill conversion), columns R..r-1 -- the ones
 * the batch has appended since its last compression -- are set to zero,
 * and in the lazily decayed form (gam != NULL, laid out by `rule` as for
 * seed_decode_step_lazy) the slot's decay product is set to 1.  Zero
 * columns add nothing to U V^T, so each slot then holds exactly the
 * handed-over state while sharing the batch's column count r: it steps with
 * the batch and is compressed with it at the batch's next compression, its
 * first window being R + W - r steps instead of W.  (Every W steps the
 * factors are compressed, SEED figures and tables, Fig. 1 (b) caption;
 * a server takes requests as they arrive, Fig. 8.)  U, V are the fp32
 * rings [batch][heads][cap][d]; requires 0 < R <= r < cap.  buf is only
 * read; calls on one batch are ordered by the caller's stream.
 */
seed_status seed_join_states(int rule, int batch, int heads, int d_k, int d_v, int cap, int R,
                             int r, int n_sel, const int *slot, const void *buf, float *a,
                             float *U, float *V, float *gam, void *stream);

/*
 * seed_state_from_dense -- convert dense states to the shallow form.
 *
 * At the end of the prefill the states are compressed to the sink plus
 * rank-R factors (SEED figures and tables, Fig. 1 (a) caption, Table 1).
 * The sink is the state's projection on vbar (Fig. 3 (b), (c)):
 *   a = S vbar / |vbar|^2,   C = S - a vbar^T,
 * and U, V (columns 0..R-1) are the rank-R truncation of C, U orthonormal.
 * S [batch][heads][d_k][d_v] and vbar [heads][d_v] are read only; a is
 * [batch][heads][d_k], U and V the usual [batch][heads][cap][d_k | d_v].
 * The caller sets r = R.  Requires 1 <= R <= min(d_k, d_v) and R <= cap;
 * R above 32 returns SEED_E_UNSUPPORTED.  Where the truncation is not
 * unique (s_R = s_{R+1}) any of the optimal ones may come back.
 */
seed_status seed_state_from_dense(int batch, int heads, int d_k, int d_v, int cap, int R,
                                  const float *S, const float *vbar,
                                  float *a, float *U, float *V, void *stream);

/*
 * seed_state_stats -- statistics of dense states, the quantities the SEED
 * figures and tables measure on model states (Fig. 3 (e), (g), (h); Fig. 12
 * (f); Fig. 13 (a), (b), (d)).  Per (request, head), with a = S vbar/|vbar|^2
 * and the content C = S - a vbar^T, rec[unit][0 .. seed_stat_fields()) is
 *   0 |S|_F^2   1 |a vbar^T|_F^2   2 |C|_F^2
 *   3 sink share |a vbar^T|_F^2 / |S|_F^2
 *   4 top share sigma_1(S)^2 / |S|_F^2
 *   5 |cos(v*, vbar)|, v* the leading right singular vector of S
 *   6, 7 the smallest k whose k largest sigma_i(C)^2 hold 90 % / 99 % of
 *        |C|_F^2 (0 for a zero content)
 *   8 the share of |C|_F^2 beyond rank R
 *   9 .. zero
 * spec_S, spec_C (float [batch][heads][d_k], optional, NULL to skip): the
 * eigenvalues of S S^T and C C^T (sigma^2 of S and C), descending, within
 * a few fp32 ulps of sigma_1^2 (Householder tridiagonalisation, bisection
 * on Sturm counts; sigma_1(S)^2 in field 4 is the Rayleigh quotient of the
 * top vector).  S and vbar are only read.
 */
int seed_stat_fields(void);
seed_status seed_state_stats(int batch, int heads, int d_k, int d_v, int R, const float *S,
                             const float *vbar, float *rec, float *spec_S, float *spec_C,
                             void *stream);

/*
 * dense_decode_step -- the dense-state baseline: one step of the head's own
 * recurrence on S (updated in place), then o = S'^T q.  The three rules are
 * the ones listed under seed_rule (the updates named in the picx.dev
 * summary, "Exact Update (Lemma 2)").  Same input conventions as
 * seed_decode_step.
 */
seed_status dense_decode_step(int rule, int batch, int heads, int d_k, int d_v, float *S,
                              const void *q, const void *k, const void *v, int in_dtype,
                              const float *g, const float *beta, float *o, void *stream);

/*
 * seed_stream_copy -- a measurement helper, not a step of the method: copies
 * `bytes` from src to dst with a plain streaming kernel (one 16-byte load
 * and store per thread, a full grid), so that the bandwidth the
 * state kernels reach can be set beside what a read-once, write-once
 * kernel gets from this device's memory.  src and dst are device buffers,
 * 16-byte aligned, not overlapping; bytes must be a multiple of 16.
 */
seed_status seed_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * seed_workspace_bytes -- bytes of caller-provided device workspace that the
 * compressions (seed_compress, seed_compress_lazy, seed_compress_h16,
 * seed_compress_sched) and the conversion (seed_state_from_dense) need for
 * `batch` requests of `heads` heads of shape d_k x d_v, capacity cap = R + W
 * and rank R.  The compression every W steps and the end-of-prefill
 * conversion (SEED figures and tables, Fig. 1 (a) and (b) captions) run in
 * one workgroup per (request, head) that keeps every intermediate (Gram
 * matrices, the small eigenproblem, the rotation) in LDS and registers, so
 * this is 0 for every shape these calls accept and none of them takes a
 * workspace argument.  Returns (size_t)-1 for a shape they reject
 * (non-positive sizes, an unsupported head shape, R > cap, cap above the
 * compiled capacity or R above 32).
 */
size_t seed_workspace_bytes(int batch, int heads, int d_k, int d_v, int cap, int R);

/* Static text for a status code. */
const char *seed_status_string(int status);

/* Thread-local description of the last failure of a call on this thread
 * ("" after a successful call). */
const char *seed_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int seed_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEED_H */
