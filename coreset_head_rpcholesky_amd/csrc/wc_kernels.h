// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// device-side flag bits (same values as WC_FLAG_* in include/wc.h)
#define WC_DFLAG_BREAKDOWN 1u
#define WC_DFLAG_NONFINITE 2u
#define WC_DFLAG_DENOM 4u
#define WC_DFLAG_DEPENDENT 8u
#define WC_DFLAG_BOUNDS 16u  // WC_DEBUG builds: an out-of-range pivot index (see wc_index_ok)

namespace wc {

// ---- resident path: one workgroup per head (n <= 256, bf16, r <= 32) ----
constexpr int kResidentRows = 256;     // n <= 256 keys
constexpr int kResidentThreads = 128;  // two waves, two consecutive key rows per thread
constexpr int kResidentR = 32;         // r <= 32 (the pivot loop is unrolled over r)
struct ResidentArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const float* u_forced;
  uint64_t seed;
  int n, m, r;
  float beta_log2e;
  uint16_t* O;        // NULL: pivot loop only
  int32_t* pivots;    // [H][r] or NULL
  float* F;           // [H][r][n] or NULL
  float* diag;        // [H][n] or NULL
  double* trace;      // [H][r+1] or NULL
  int32_t* rank;      // [H]
  uint32_t* flags;    // [H]
  float* W;           // [H][r][dv+1] or NULL
};
hipError_t launch_resident_64_64(const ResidentArgs& a, int heads, hipStream_t st);
hipError_t launch_resident_64_128(const ResidentArgs& a, int heads, hipStream_t st);
hipError_t launch_resident_128_64(const ResidentArgs& a, int heads, hipStream_t st);
hipError_t launch_resident_128_128(const ResidentArgs& a, int heads, hipStream_t st);
inline hipError_t launch_resident(const ResidentArgs& a, int heads, int d, int dv, hipStream_t st) {
  if (d == 64) return dv == 64 ? launch_resident_64_64(a, heads, st) : launch_resident_64_128(a, heads, st);
  return dv == 64 ? launch_resident_128_64(a, heads, st) : launch_resident_128_128(a, heads, st);
}

// ---- streaming pivot loop: one launch per pivot step over all heads ----
struct StreamRpcArgs {
  const void* K;        // [H][n][d], float or bf16
  int bf16;
  const float* u_forced;
  uint64_t seed;
  float* uniforms;      // [H][r]: u_forced, or filled from Philox before the first step
  int H, n, d, r;
  int rows;             // rows per workgroup: 256, or 1024 when n % 4 == 0
  int nblk;             // row blocks per head, ceil(n / rows) <= 4096
  float beta_log2e;
  float* F;             // [H][r][n]
  float* diag0;         // [H][n] double-buffered residual diagonal
  float* diag1;
  double* part0;        // [H][nblk] double-buffered block masses
  double* part1;
  int32_t* pivots;      // [H][r]
  double* trace;        // [H][r+1] or NULL
  int32_t* rank;        // [H]
  uint32_t* flags;      // [H]
  float* diag_out;      // [H][n] or NULL
};
constexpr int kStreamThreads = 256;
hipError_t launch_rpc_stream(const StreamRpcArgs& a, hipStream_t st);

// ---- block pivot selection: b candidates per round (the fields of the streaming loop plus) ----
constexpr int kBlockDraws = 4;  // candidates drawn per pivot slot at most
struct BlockRpcArgs {
  StreamRpcArgs s;      // K, residual and block masses (rows, nblk), F, pivots, rank (slots
                        // filled so far), ...; s.uniforms holds kBlockDraws r per head
  int b;                // candidates per round: 16, 32 or 64, dividing r
  float tol;            // relative residual at or below which a candidate is passed over
  int32_t* cand;        // ws [H][b]
  int32_t* slot;        // ws [H][b]     slot a candidate fills, or -1
  float* G;             // ws [H][b][n]  candidate columns minus what F explains
  float* M;             // ws [H][b][b]  inverse factor of the kept part of the candidate block
  int32_t* rounds;      // ws [H]        rounds applied so far (the residual's buffer parity)
  float* FS;            // ws [H][r][b]  factor rows at the round's candidates, by factor column
};
hipError_t launch_rpc_block(const BlockRpcArgs& a, hipStream_t st);

// ---- weights: W = L^{-T} F^T [V, 1] ----
struct WeightsArgs {
  const void* V;          // [H][n][dv]
  int bf16;
  int H, n, dv, r;
  const float* F;         // [H][r][n]
  const int32_t* pivots;  // [H][r]
  const int32_t* rank;    // [H]
  float* L;               // ws [H][r][r]   L[t][j] = F[j][s_t]
  float* Xpart;           // ws [H][nchunk][r][dv+1]
  int nchunk, chunk_rows;
  float* X;               // ws [H][r][dv+1]
  float* W;               // out [H][r][dv+1]
  float* Minv;            // ws [H][r/64][64][64] inverses of L's diagonal blocks, or NULL: the
                          // blocked back substitution (r a multiple of 64) instead of trisolve
  uint32_t* flags;        // [H] or NULL: WC_DFLAG_BOUNDS for an out-of-range pivot (WC_DEBUG)
};
hipError_t launch_weights(const WeightsArgs& a, hipStream_t st);

// ---- bins: per-bin selection and weights ran on heads * B sub-heads; fold them per head ----
struct BinsArgs {
  int H, B, nb, rb;              // heads, bins, keys and pivots per bin
  const int32_t* piv_sub;        // [H*B][rb], -1 after a bin's breakdown
  const int32_t* rank_sub;       // [H*B]
  const uint32_t* flags_sub;     // [H*B]
  int32_t* pivots;               // out [H][B*rb]: key index within the head, or -1
  int32_t* rank;                 // out [H]: pivots taken over all bins
  uint32_t* flags;               // out [H]: OR over the bins
  int32_t* rank_slots;           // out [H]: B*rb, the slots the attention scans
};
hipError_t launch_bins_combine(const BinsArgs& a, hipStream_t st);

// ---- attend: O = (exp(beta Q K_S^T) W)[:, :dv] / (...)[:, dv] ----
struct AttendArgs {
  const void* Q;          // [H][m][d]
  const void* K;          // [H][n][d]
  const void* V;          // [H][n][dv] (the all-keys preparation only)
  int bf16;
  int H, n, m, d, dv, r;
  float beta_log2e;
  const int32_t* pivots;
  const int32_t* rank;
  const float* W;         // [H][r][dv+1]
  uint16_t* KSh;          // ws [H][rp*d]     coreset keys, bf16 hi, tile-major (rp = attend_rows(r))
  uint16_t* KSl;          // ws [H][rp*d]     bf16 lo (fp32 inputs only)
  uint16_t* Wph;          // ws [H][dv*rp]    permuted W^T, bf16 hi, tile-major
  uint16_t* Wpl;          // ws [H][dv*rp]    bf16 lo (fp32 inputs only)
  float* Wden;            // ws [H][rp]       W[:, dv]
  uint16_t* Wdh;          // ws [H][rp]       W[:, dv] in bf16, permuted like the columns of W^T
  float* Ypart;           // ws [H][nsplit][m][dv+1] partial sums when nsplit > 1
  int nsplit;
  void* O;                // [H][m][dv]
  uint32_t* flags;        // [H]
  float* Yout;            // NULL, or [H][yrows][dv+1]: the unnormalised Y in fp32 instead of O
  int yrows;
  int ldrows;             // staged rows per head (0: attend_rows(r)); a cache uses its capacity
  int scan_rows;          // rows the attention scans (0: all staged rows); rows at or past it get
                          // zero probability whatever the staged row holds
  int row0;               // first row written by the append staging
};
// coreset rows as the attention kernels store them: r rounded up to whole 128-row blocks
// (padding rows carry zero weight)
__host__ __device__ inline int attend_rows(int r) { return (r + 127) & ~127; }
__host__ __device__ inline int staged_rows(const AttendArgs& a) { return a.ldrows ? a.ldrows : attend_rows(a.r); }
__host__ __device__ inline int scanned_rows(const AttendArgs& a) {
  return a.scan_rows ? attend_rows(a.scan_rows) : staged_rows(a);
}
hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
// The same attention with every key as a coreset row and W = [V, 1] (r = n): stage the keys
// and values, then run the attention proper (normally with Yout set, giving
// Y = exp(beta Q K^T) [V, 1]).
hipError_t launch_attend_all_keys(const AttendArgs& a, hipStream_t st);
// Staging only (the coreset rows into the staged layout, every staged row written).
hipError_t launch_attend_prep(const AttendArgs& a, hipStream_t st);
// Exact rows: key j of K with weight row [v_j, 1], written at staged row row0 + j (n rows).
hipError_t launch_attend_append(const AttendArgs& a, hipStream_t st);
// The attention proper over already staged rows (no staging).
hipError_t launch_attend_core(const AttendArgs& a, hipStream_t st);
// Decode: at most kDecodeMaxQueries bf16 queries per head over staged rows [0, scan_rows),
// kDecodeWaves 64-row chunks per workgroup; with more than one workgroup per head the fp32
// partials go to Ypart [H][decode_splits(scan_rows)][m][dv+1] and a reduction writes O.
constexpr int kDecodeWaves = 16;
constexpr int kDecodeMaxQueries = 8;
__host__ __device__ inline int decode_splits(int rows) {
  const int chunks = (rows + 63) / 64;
  return (chunks + kDecodeWaves - 1) / kDecodeWaves;
}
hipError_t launch_decode(const AttendArgs& a, hipStream_t st);

// ---- union weights of the divide-and-conquer forward: H_SS^+ X over all bins' pivots ----
struct UnionArgs {
  const void* K;          // [H][n][d]
  int bf16;
  int H, n, d, dv, r;
  int rp;                 // r rounded up to 64
  float beta;             // 1/sqrt(d)
  float tol;              // relative residual at or below which a point is left out
  const int32_t* pivots;  // [H][r]: key index, or -1 for an empty slot
  void* Qs;               // ws [H][r][d]  coreset keys as rows (input dtype), zero for empty slots
  float* A;               // ws [H][rp][rp] H_SS, factored in place (lower blocks)
  float* Hd;              // ws [H][rp]     diagonal of H_SS
  float* M;               // ws [H][rp/64][64][64] inverses of the kept parts of the diagonal blocks
  float* X;               // ws [H][rp][dv+1] H_{S,:}[V, 1] in (rows < r), substituted in place
  float* W;               // out [H][r][dv+1]
  uint32_t* flags;        // [H]: WC_DFLAG_DEPENDENT when a point of a valid slot is left out
};
// out[h][j] = pivots[h][j] for j < rank[h], else -1 (the slots of wc_weights_keys)
hipError_t launch_union_mask(const int32_t* pivots, const int32_t* rank, int32_t* out, int H, int r, hipStream_t st);
hipError_t launch_union_gather(const UnionArgs& a, hipStream_t st);  // fills Qs
hipError_t launch_union_solve(const UnionArgs& a, hipStream_t st);   // A, Hd, M from Qs; X -> W
// The blocked back substitution alone: W = L^{-T} X from the lower factor L (in A, leading
// dimension rp, a multiple of 64), the inverses M of its diagonal blocks and X (overwritten).
hipError_t launch_union_back(const UnionArgs& a, hipStream_t st);

// ---- key centring: Kc = K - mean of the head's keys (fp64 mean, input-precision result) ----
struct CenterArgs {
  const void* K;          // [H][n][d]
  int bf16;
  int H, n, d;
  int nblk;               // center_blocks(n)
  double* part;           // ws [H][nblk][d]
  double* mean;           // ws [H][d]
  void* Kc;               // ws [H][n][d], input dtype
};
constexpr int kCenterRows = 1024;  // key rows per workgroup of the column sums
inline int center_blocks(int n) { return (n + kCenterRows - 1) / kCenterRows; }
hipError_t launch_center(const CenterArgs& a, hipStream_t st);

}  // namespace wc
