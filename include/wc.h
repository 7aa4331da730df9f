/*
 * wc.h — C ABI of the WildCat hot path on AMD Instinct MI355X (gfx950).
 *
 * WildCat approximates softmax attention by attending only over a small weighted coreset of
 * the keys (page "WildCat: Near-Linear Attention in Theory and Practice",
 * gptget.net/papers/2602.10056, Abstract).  Per head the path is
 *
 *   1. coreset selection by randomly pivoted Cholesky (RPCholesky) on the kernel matrix
 *      H = exp(beta K K^T), beta = 1/sqrt(d), each pivot drawn from the residual diagonal
 *      (gist.science/de/paper/2602.10056, "Methodik", part 1);
 *   2. Nystroem weights W = H_SS^{-1} H_{S,:} [V, 1]  (r x (dv+1)); the first dv columns are
 *      the pages' compressed values V_S = W_pages V, the last is W_pages 1, the softmax
 *      normaliser (same page, "Methodik", part 2);
 *   3. attention of every query over the weighted coreset:
 *      Y = exp(beta Q K_S^T) W,  O = Y[:, :dv] / Y[:, dv].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - `wc_problem` is a host pointer.  Every other pointer is a DEVICE pointer (memory of the
 *    current HIP device) and must be 16-byte aligned.  The caller owns all memory; the
 *    library never allocates, frees or retains device memory, and keeps no mutable global
 *    state, so calls are re-entrant.  Inputs are never modified; outputs must not alias
 *    inputs or the workspace.
 *  - Layouts are dense row-major: Q [heads][m][d], K [heads][n][d], V [heads][n][dv],
 *    O [heads][m][dv] in the problem's dtype; F [heads][r][n] float (column t of the n x r
 *    factor is contiguous); W [heads][r][dv+1] float; pivots [heads][r] int32;
 *    u_forced [heads][r] float; diag [heads][n] float; trace [heads][r+1] double;
 *    rank [heads] int32; flags [heads] uint32.
 *  - `heads` counts every (batch, head) pair.  `bins` selects divide-and-conquer selection in
 *    wc_forward (see there); 0 or 1 everywhere else.  `options` holds WC_OPT_* bits (any
 *    other bit is WC_ERR_INVALID_ARG).  Supported: d, dv in {64, 128};
 *    dtype WC_F32 or WC_BF16; 1 <= r <= min(n, 4096); n, m >= 1 (m may be 0 for
 *    wc_attend/wc_forward: nothing is written then); heads == 0 is a no-op.
 *  - Every call validates its arguments on the host BEFORE any HIP call; on failure it
 *    returns a non-zero status and enqueues nothing.  On success the work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and the call returns without
 *    waiting.  A failed launch returns WC_ERR_DEVICE.  No call throws.
 *  - Numeric conditions found on the device are reported per head, readable after the
 *    stream is synchronised: rank[h] = number of pivots actually taken, and flags[h]:
 *       WC_FLAG_BREAKDOWN  rank < r: the residual trace or a pivot's residual reached <= 0
 *       WC_FLAG_NONFINITE  a non-finite value reached the pivot loop
 *       WC_FLAG_DENOM      some query row had a normaliser Y[:, dv] <= 0
 *       WC_FLAG_DEPENDENT  (bins > 1) the union weights left out a coreset point that is
 *                          numerically dependent on earlier ones (see wc_forward)
 *       WC_FLAG_BOUNDS     (debug library libwc_debug.so only) a pivot index read from device
 *                          memory lay outside [0, n); the slot was treated as empty.  The
 *                          regular library does not check pivot indices it is handed.
 *    After a breakdown pivots[rank..r-1] = -1, F columns rank..r-1 = 0, and weights and
 *    attention use the first rank pivots only.
 *  - Workspace: `ws` must hold at least wc_workspace_bytes() bytes for the same problem.
 */
#ifndef WC_H_
#define WC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WC_ABI_VERSION 9

typedef enum {
  WC_OK = 0,
  WC_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, r > n, ... */
  WC_ERR_UNSUPPORTED = 2, /* d, dv or dtype outside the supported set, r > 4096 */
  WC_ERR_WORKSPACE = 3,   /* ws NULL or smaller than wc_workspace_bytes() */
  WC_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
} wc_status;

typedef enum { WC_F32 = 0, WC_BF16 = 1 } wc_dtype;

enum {
  WC_FLAG_BREAKDOWN = 1u,
  WC_FLAG_NONFINITE = 2u,
  WC_FLAG_DENOM = 4u,
  WC_FLAG_DEPENDENT = 8u,
  WC_FLAG_BOUNDS = 16u
};

/* wc_problem.options bits */
enum {
  WC_OPT_BIN_WEIGHTS = 1u, /* bins > 1: per-bin weights instead of weights over the union */
  WC_OPT_CENTER_KEYS = 2u  /* wc_forward only: run on the centred keys (see wc_forward) */
};

typedef struct {
  int32_t heads; /* batch * heads, each an independent problem */
  int32_t n;     /* keys (and values) per head */
  int32_t m;     /* queries per head */
  int32_t d;     /* key/query width: 64 or 128 */
  int32_t dv;    /* value width: 64 or 128 */
  int32_t r;     /* coreset size (pivot steps) */
  int32_t dtype; /* wc_dtype of Q, K, V and O */
  int32_t bins;  /* 0 or 1: one bin; B > 1: divide-and-conquer selection (wc_forward only) */
  int32_t options; /* OR of WC_OPT_* bits; 0 for the defaults */
  int32_t pivot_block; /* 0 or 1: one pivot per step; b in {16, 32, 64}: b candidates per round
                          (wc_rpcholesky, wc_forward, wc_compress; see wc_rpcholesky) */
} wc_problem;

/* ABI version of the loaded library (WC_ABI_VERSION it was built with). */
int32_t wc_abi_version(void);

/* Static description of a status code; never NULL. */
const char* wc_status_string(wc_status s);

/* Workspace bytes needed by wc_rpcholesky, wc_weights, wc_attend and wc_forward for this
 * problem (one size serves all four).  *bytes is set on WC_OK only. */
wc_status wc_workspace_bytes(const wc_problem* p, size_t* bytes);

/* Randomly pivoted partial Cholesky of H = exp(beta K K^T) with r pivots per head
 * (gist.science/de/paper/2602.10056, "Methodik" part 1: partial Cholesky of the kernel
 * matrix, pivot sampled from the residual diagonal).
 *
 * Step t: p = max(diag, 0); T = sum p (fp64); s = min{i : C_i > u_t T} for the running sum C
 * of p; g = H[:, s] - F[:, :t] F[s, :t]^T; F[:, t] = g / sqrt(g[s]); diag -= F[:, t]^2;
 * diag[s] = 0.
 *   K        in   [heads][n][d], dtype
 *   u_forced in   [heads][r] float in [0,1), or NULL: then u_t comes from Philox4x64-10
 *                 with counter (t, head, 0, 0) and key (seed, 0), u = (x0 >> 40) * 2^-24
 *   pivots   out  [heads][r]
 *   F        out  [heads][r][n]
 *   diag     out  [heads][n] final residual diagonal, or NULL
 *   trace    out  [heads][r+1]: trace[t] = T before step t, trace[r] after the last, or NULL
 *   rank, flags out [heads]                                                              */
/* pivot_block = b > 1 (b in {16, 32, 64} dividing r, or r / bins with bins): b candidate
 * pivots per round.  The pages leave a remedy for the sequential pivot selection (an
 * oversampling mechanism) to future work (gist.science/de/paper/2602.10056, "Bedeutung und
 * Ansprueche"); this is the block variant of randomly pivoted Cholesky, oversampled until the
 * slots are full.  Round k draws its b candidates from the residual at the start of the round
 * (u_forced[h][k b + j], or Philox with counter (k b + j, head)), forms their columns
 * together, G = H[:, S] - F F[S, :]^T (F read once per round), then takes them in order:
 * candidate j enters the next free slot when its residual after the round's earlier accepted
 * candidates exceeds 2^-12 H_ss, and is passed over otherwise (an index drawn again, or one
 * dependent on them).  Rounds go on until the r slots are full or 4 r candidates are drawn,
 * so u_forced holds 4 r values per head ([heads][4 r]); running out of draws (or of mass) is a
 * breakdown with rank < r.  The pivots fill slots 0 .. rank-1 as in the one-pivot loop, and
 * F[S, :] is lower triangular, so wc_weights and wc_attend take them as they are.  trace[t]
 * holds the total mass before the round that started with t slots full, trace[r] the total
 * after the last round, other entries 0.  With bins, each bin does this on its own keys and
 * draws u_forced[h][4 s0 .. 4 s1) for its slots [s0, s1).                                  */
wc_status wc_rpcholesky(const wc_problem* p, const void* K, const float* u_forced,
                        uint64_t seed, int32_t* pivots, float* F, float* diag, double* trace,
                        int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes,
                        void* stream);

/* Nystroem weights W = H_SS^{-1} H_{S,:} [V, 1] for the first rank[h] pivots
 * (gist.science/de/paper/2602.10056, "Methodik" part 2: W = h(K_S,K_S)^+ h(K_S,K), V_S = W V).
 * Takes the factor F of wc_rpcholesky in place of the keys: the factor yields the weights
 * without a second pass over the keys and is the more accurate order in fp32.  Pivots that
 * come without their factor take wc_weights_keys below (keys in).  With
 * L = F[S, :] (lower triangular, L L^T = H_SS) and H_{:,S} = F L^T, W = L^{-T} F^T [V, 1].
 *   V             in  [heads][n][dv], dtype
 *   pivots, rank  in  as returned by wc_rpcholesky
 *   F             in  [heads][r][n], the factor returned by wc_rpcholesky for these pivots
 *   W             out [heads][r][dv+1]; rows rank..r-1 are zero                            */
wc_status wc_weights(const wc_problem* p, const void* V, const int32_t* pivots,
                     const int32_t* rank, const float* F, float* W, void* ws, size_t ws_bytes,
                     void* stream);

/* Nystroem weights from the keys, for any pivots (gist.science/de/paper/2602.10056, "Methodik"
 * part 2: W = h(K_S,K_S)^+ h(K_S,K)): W = H_SS^+ H_{S,:} [V, 1] over the slots j < rank[h]
 * (slots past the rank, and pivots -1, are empty: zero weight rows).  H_{S,:} [V, 1] comes
 * from one pass of the attention kernels over all n keys, and the pseudo-inverse is the
 * Cholesky of H_SS in slot order that leaves out every point whose residual is at most
 * 2^-12 H_jj (a repeated pivot, or one numerically in the span of the earlier ones): its weight
 * row is zero and WC_FLAG_DEPENDENT is OR-ed into flags[h].  For distinct, independent pivots
 * (those of wc_rpcholesky) this is the inverse, and W equals wc_weights' up to rounding.
 * Precision: bf16 problems form H_{S,:} [V, 1] with bf16 probabilities (fp32 sums), so its
 * rounding reaches W amplified by the conditioning of H_SS.  Pivot indices must lie in
 * [0, n) or be -1; the debug library flags others (WC_FLAG_BOUNDS) and treats them as empty.
 *   K             in  [heads][n][d], dtype
 *   V             in  [heads][n][dv], dtype
 *   pivots        in  [heads][r] key indices or -1;  rank in [heads]
 *   W             out [heads][r][dv+1]
 *   flags         in/out [heads]: WC_FLAG_DEPENDENT is OR-ed in
 *   ws            at least wc_weights_keys_workspace_bytes() bytes (its own size: the all-keys
 *                 pass and the blocked solve, not the other entry points' workspace)           */
wc_status wc_weights_keys_workspace_bytes(const wc_problem* p, size_t* bytes);
wc_status wc_weights_keys(const wc_problem* p, const void* K, const void* V, const int32_t* pivots,
                          const int32_t* rank, float* W, uint32_t* flags, void* ws, size_t ws_bytes,
                          void* stream);

/* Attention of every query over the weighted coreset (page gptget.net/papers/2602.10056,
 * Abstract: attend only over a small weighted coreset): Y = exp(beta Q K_S^T) W,
 * O = Y[:, :dv] / Y[:, dv], with K_S the keys at the first rank[h] pivots.  Precision: bf16
 * problems round the probabilities and W (the normaliser column included) to bf16 on the
 * matrix cores with fp32 sums, so a query row whose normaliser condition number
 * sum |P| |W[:, dv]| / |Y[:, dv]| is kappa carries a relative error of about 2^-8 (1 + kappa);
 * fp32 problems use hi + lo bf16 splits (about 2^-16 relative).
 *   Q           in  [heads][m][d], dtype
 *   K, pivots, rank, W   in  as above
 *   O           out [heads][m][dv], dtype
 *   flags       in/out [heads]: WC_FLAG_DENOM is OR-ed in                                   */
wc_status wc_attend(const wc_problem* p, const void* Q, const void* K, const int32_t* pivots,
                    const int32_t* rank, const float* W, void* O, uint32_t* flags, void* ws,
                    size_t ws_bytes, void* stream);

/* The whole forward: wc_rpcholesky, wc_weights and wc_attend in one call (the factor and the
 * weights live in the workspace).  pivots may be NULL; rank and flags are required.
 *
 * bins = B > 1 (divide-and-conquer selection, gist.science/de/paper/2602.10056, "Methodik"
 * part 1, efficiency: B bins processed in parallel at O(n r^2/B^3 + n r d/B^2)): B must divide
 * n and r.  Bin b holds the keys [b n/B, (b+1) n/B) and the pivot slots [b r/B, (b+1) r/B);
 * each bin runs the pivot loop on its keys (u_forced[h][slot], or Philox with counter
 * (t, h B + b, 0, 0) for the bin's step t).  The coreset K_S is the union of the bins'
 * pivots in slot order, and its weights ("Methodik" part 2) are
 *   default             W = H_SS^+ H_{S,:} [V, 1] over all n keys.  The pseudo-inverse is a
 *                       Cholesky of H_SS in slot order that leaves out every point whose
 *                       residual is at most 2^-12 H_jj (numerically in the span of the
 *                       earlier points; its weight row is zero and WC_FLAG_DEPENDENT is set).
 *                       For distinct keys nothing is left out and it is the inverse.
 *   WC_OPT_BIN_WEIGHTS  each bin's keys get their own weights on that bin's coreset,
 *                       W_b = H_{S_b S_b}^{-1} H_{S_b, bin b} [V_b, 1]: cheaper, less accurate.
 * Every query attends over the union.  pivots[h][j] is the key index within the head, or -1
 * for a slot its bin left empty after a breakdown (no longer only at the end); rank[h] counts
 * the pivots taken over all bins; flags are OR-ed over the bins.  The other entry points take
 * bins <= 1 (WC_ERR_UNSUPPORTED otherwise): their per-bin view is the problem with heads * B
 * heads of n/B keys and r/B pivots.
 *
 * WC_OPT_CENTER_KEYS ("Methodik" part 3: softmax attention is invariant under a global shift
 * of the keys, which are re-centred by their mean): every step runs on Kc = K - mean of the
 * head's keys, the mean a fixed-order fp64 sum, Kc formed in fp64 and stored in the input
 * precision (bf16 through fp32, round to nearest even).  Queries are not shifted: the factor
 * exp(-beta q.mean) is common to a query's numerator and normaliser.  The pivots then refer
 * to the centred keys (same indices).  Needs wc_workspace_bytes() of the problem with the
 * option set.  The other entry points return WC_ERR_UNSUPPORTED for it.                      */
wc_status wc_forward(const wc_problem* p, const void* Q, const void* K, const void* V,
                     const float* u_forced, uint64_t seed, void* O, int32_t* pivots,
                     int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes, void* stream);

/* wc_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same arguments and results as
 * wc_forward, with no workspace argument.  The workspace is a device array inside the library,
 * WC_NOALLOC_MAX_WORKSPACE bytes, which every device the library runs on holds until the
 * process ends.  A problem whose wc_workspace_bytes() exceeds it returns WC_ERR_WORKSPACE
 * and enqueues nothing.  The call allocates and frees nothing.  All calls on one device share
 * that device's array: calls that overlap on one device (different streams, or host threads)
 * race on it and must be ordered by the caller.                                              */
#define WC_NOALLOC_MAX_WORKSPACE ((size_t)256 << 20)
wc_status wc_forward_noalloc(const wc_problem* p, const void* Q, const void* K, const void* V,
                             const float* u_forced, uint64_t seed, void* O, int32_t* pivots,
                             int32_t* rank, uint32_t* flags, void* stream);

/* ---- COMPRESSKV: a compressed KV cache and decode over it ----------------------------------
 * gist.science/de/paper/2602.10056, "Zentrale Beitraege": a COMPRESSKV module shrinks the KV
 * cache from Theta(n d) to O(r d).  A cache holds, per head, up to `capacity` rows; a row is a
 * key with a weight row of dv+1 floats.  wc_compress fills rows [0, r) with the coreset of a
 * prefix (K_S and the weights W of wc_forward, same pivots, bins and options) and zeroes the
 * rest.  Tokens that come later are appended as exact rows (key k, weights [v, 1]), a reading
 * the pages leave open: their contribution exp(beta q k) [v, 1] is exactly that of softmax
 * attention.  wc_decode attends queries over rows [0, rows):
 *     Y = sum over rows of exp(beta q k_row) w_row,   O = Y[:dv] / Y[dv].
 * The cache is opaque device memory of wc_cache_bytes() bytes (16-byte aligned), laid out for
 * the attention kernels: keys as bf16 (hi and lo parts for fp32 problems), weights as bf16
 * (hi and lo for fp32) with the normaliser column also in fp32.  `p` gives heads, d, dv and
 * dtype for every cache call, n and r for wc_compress, m for wc_decode; the same capacity
 * must be passed to every call on one cache.  wc_decode reads rows [0, rows) only: whatever
 * rows at or past `rows` hold (later appends, stale rows) takes no part in the output.       */

/* Bytes of a cache with `capacity` rows per head (capacity >= 1). */
wc_status wc_cache_bytes(const wc_problem* p, int32_t capacity, size_t* bytes);

/* Compress the prefix K, V ([heads][n][d], [heads][n][dv]) into rows [0, r) of `cache`
 * (capacity >= r).  u_forced, seed, pivots, rank, flags and the workspace are those of
 * wc_forward for the same problem (wc_workspace_bytes); m is ignored.  A slot left empty
 * (pivot -1) or a point left out of the union weights is a row of weight zero.             */
wc_status wc_compress(const wc_problem* p, const void* K, const void* V, const float* u_forced,
                      uint64_t seed, void* cache, int32_t capacity, int32_t* pivots,
                      int32_t* rank, uint32_t* flags, void* ws, size_t ws_bytes, void* stream);

/* Append `count` exact rows per head: key j of K_new [heads][count][d] with weights
 * [V_new[j], 1] ([heads][count][dv]) at row row0 + j; row0 + count <= capacity.           */
wc_status wc_cache_append(const wc_problem* p, const void* K_new, const void* V_new,
                          int32_t count, int32_t row0, void* cache, int32_t capacity,
                          void* stream);

/* Workspace of wc_decode for p->m queries per head over `rows` rows (may be 0 bytes). */
wc_status wc_decode_workspace_bytes(const wc_problem* p, int32_t rows, size_t* bytes);

/* Attention of Q [heads][m][d] over rows [0, rows) of the cache (1 <= rows <= capacity);
 * O [heads][m][dv] in the problem's dtype; WC_FLAG_DENOM is OR-ed into flags [heads].
 * bf16 problems with m <= 8 run a decode kernel (one workgroup per 1024 rows per head and
 * query, fp32 probabilities and normaliser, a split reduction past 1024 rows); others run the
 * attention kernels with the rows split over workgroups.                                    */
wc_status wc_decode(const wc_problem* p, const void* Q, const void* cache, int32_t capacity,
                    int32_t rows, void* O, uint32_t* flags, void* ws, size_t ws_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------------------
 * Calibration (a measurement helper, not a step of the method).  The rooflines of the hot
 * path are quoted against the datasheet peaks of the part (HBM 8 TB/s; dense matrix cores:
 * bf16 2.5 PFLOP/s, fp32 157.3 TFLOP/s, both at 2.4 GHz).  These kernels measure what the part
 * attains on the same operations, so that the attainable rates can be reported beside them:
 *   WC_CAL_READ       reads `bytes` of src (16-byte nontemporal loads, sixteen in flight
 *                     per lane, 8192 workgroups of 256 threads); dst receives one XOR word
 *                     per wave (128 KiB);
 *   WC_CAL_COPY       copies `bytes` of src to dst (the ranges must not overlap);
 *   WC_CAL_MFMA_BF16  512 workgroups of 4 waves (two per SIMD) each run `iters` rounds of 8
 *                     independent v_mfma_f32_32x32x16_bf16 on register operands, 2^15 flops
 *                     each; all operands are 1, so dst[w] (one float per wave, 8 KiB) is
 *                     2048 iters exactly while that is below 2^24;
 *   WC_CAL_MFMA_F32   the same with v_mfma_f32_32x32x2_f32 (2^12 flops each); dst[w] =
 *                     256 iters.
 * src and dst are 16-byte aligned device pointers (src unused by the MFMA kinds; bytes a
 * nonzero multiple of 16 for READ and COPY; iters >= 1 for the MFMA kinds).  clocks is NULL
 * or a device pointer to 4 uint64: the shader clock (s_memtime) and the 100 MHz reference
 * clock (s_memrealtime) read by workgroup 0 at its start and its end, MFMA kinds only.  An
 * unknown kind or a bad argument returns WC_ERR_INVALID_ARG before any HIP call; the work is
 * enqueued on `stream` otherwise.                                                          */
typedef enum {
  WC_CAL_READ = 0,
  WC_CAL_COPY = 1,
  WC_CAL_MFMA_BF16 = 2,
  WC_CAL_MFMA_F32 = 3
} wc_cal_kind;
#define WC_CAL_RESULT_BYTES 131072 /* dst size that every kind but COPY needs */
wc_status wc_calibrate(int32_t kind, const void* src, void* dst, size_t bytes, int32_t iters,
                       uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* WC_H_ */
