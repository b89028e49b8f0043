// Internal constants shared by the host checks and the HIP kernels.
#ifndef CODA_INTERNAL_H
#define CODA_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

namespace coda {

// Block tile of every GEMM: 256 x 256 outputs, K step 64, 8 waves in two
// groups of four; each group owns 128 rows, each wave a 128 x 64 sub-tile.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kWaveTileM = 128;
constexpr int kWaveTileN = 64;
constexpr int kThreads = 512;

// K0, D and N must be multiples of this: the K step (every contraction runs whole K steps) and the
// wave tile width (each wave's 64 output columns lie wholly inside or wholly past the last column).
constexpr int64_t kDimQuantum = 64;
// Largest accepted K0 / D / N and M (keeps every per-tile buffer offset < 2^31 and a
// one-block-per-row launch of 512-thread blocks within 2^32 work-items); each GEMM's
// grid is also checked against that limit.
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxRows = int64_t(1) << 22;

// Row block of the unfused RMSNorm-backward kernel (its dgamma partial granularity).
constexpr int kUnfusedBwdRows = 32;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Column count of the forward's sum-of-squares partials P[M, ceil(D / kBN)]: one per row and
// 256-column tile of GEMM0 (its four waves' 64-column sums added in the block).
inline int64_t ssq_cols(int64_t D) { return ceil_div(D, kBN); }
// GEMM1's epilogue combines r from P itself, with no separate combine launch, when
//   * a wave's 128 rows of partials fit its 16 KB LDS staging area: at most 32 per row, D <= 8192;
//   * GEMM1 has at most two waves of tiles on the 256 CUs: each tile pays the partials' DMA and the
//     combine again (measured at the 8B shape: about 2.7 us per wave of tiles, against about 1 us for
//     the separate launch in stream), so larger GEMMs keep the separate kernel.
constexpr int64_t kFoldedCombineMaxCols = 32;
constexpr int64_t kFoldedCombineMaxTiles = 512;
inline bool fwd_folds_combine(int64_t M, int64_t D, int64_t N) {
  return ssq_cols(D) <= kFoldedCombineMaxCols && ceil_div(M, kBM) * ceil_div(N, kBN) <= kFoldedCombineMaxTiles;
}
// Column count of the SwiGLU backward's s partials Ps[M, (N / 2) / kWaveTileN].
inline int64_t swiglu_s_cols(int64_t N) { return (N / 2) / kWaveTileN; }
// Column count of the cross-entropy tile statistics Pml[M, V / kWaveTileN] (float2).
inline int64_t ce_stat_cols(int64_t V) { return V / kWaveTileN; }
// Cross-entropy forward workspace: Pml, then the target logits [M] fp32.
inline size_t ce_fwd_ws(int64_t M, int64_t V) {
  return align256(size_t(M) * size_t(ce_stat_cols(V)) * 8) + align256(size_t(M) * 4);
}
// Unfused cross-entropy workspace: the fp32 logits [M, V].
inline size_t unfused_ce_ws(int64_t M, int64_t V) { return align256(size_t(M) * size_t(V) * 4); }
// Row count of the fused backward's dgamma partials Pg[ceil(M / kWaveTileM), D].
inline int64_t dgamma_rows(int64_t M) { return ceil_div(M, kWaveTileM); }

// Split-K of the data-gradient GEMM G = dY @ W1^T (contraction over N) when its
// ceil(M / 256) * D / 256 tiles cannot fill the chip (few rows: a data-parallel
// shard): S slices of kslice columns each (a multiple of the K step, at least four
// steps), at most 8, aiming at one tile per CU. S = 1: no split.
struct KSplit {
  int64_t S, kslice;
};
inline KSplit dgrad_split(int64_t M, int64_t D, int64_t N) {
  const int64_t tiles = ceil_div(M, kBM) * ceil_div(D, kBN);
  int64_t S = ceil_div(256, tiles);
  if (S > 8) S = 8;
  if (S > N / kBK / 4) S = N / kBK / 4;
  if (tiles >= 192 || S < 2) return {1, 0};
  const int64_t kslice = ceil_div(ceil_div(N, S), kBK) * kBK;
  return {ceil_div(N, kslice), kslice};
}
// Split-K of GEMM0 (contraction over K0), by the same rule. The workspace is sized
// without K0 for S_max = min(ceil(256 / tiles), 8) slices; a call uses
// S = min(S_max, K0 / 256) of them (at least four K steps each).
inline int64_t gemm0_split_max(int64_t M, int64_t D) {
  const int64_t tiles = ceil_div(M, kBM) * ceil_div(D, kBN);
  if (tiles >= 192) return 1;
  const int64_t S = ceil_div(256, tiles);
  return S > 8 ? 8 : S;
}
inline KSplit gemm0_split(int64_t M, int64_t K0, int64_t D) {
  int64_t S = gemm0_split_max(M, D);
  if (S > K0 / kBK / 4) S = K0 / kBK / 4;
  if (S < 2) return {1, 0};
  const int64_t kslice = ceil_div(ceil_div(K0, S), kBK) * kBK;
  return {ceil_div(K0, kslice), kslice};
}
// Device scratch of the no-allocation forward (coda_fwd_noalloc): its partials P [M, ceil(D / 256)] fp32.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
// Fused forward workspace: the sums of squares P [M, ceil(D / 256)], then (split-K only) the
// fp32 partial products [S_max, M, D].
inline size_t fwd_ws_p(int64_t M, int64_t D) { return align256(size_t(M) * size_t(ssq_cols(D)) * 4); }
inline size_t fwd_ws(int64_t M, int64_t D) {
  const int64_t S = gemm0_split_max(M, D);
  return fwd_ws_p(M, D) + (S > 1 ? align256(size_t(S) * size_t(M) * size_t(D) * 4) : 0);
}
// Row group of the split-K reduction kernel (its dgamma partials have ceil(M / 8) rows):
// small enough that a shard's rows give the kernel several blocks per CU.
constexpr int kSplitRows = 8;
inline int64_t bwd_pg_rows(int64_t M, int64_t D, int64_t N) {
  return dgrad_split(M, D, N).S > 1 ? ceil_div(M, kSplitRows) : dgamma_rows(M);
}
// Fused backward workspace: bf16(r g) transposed, [D, gr_cols(M)], then the dgamma partials Pg, then
// (split-K only) the fp32 partial products [S, M, D].
// Rows of the transposed bf16(r g): M rounded up to the K step (the pad is zero).
inline int64_t gr_cols(int64_t M) { return ceil_div(M, kBK) * kBK; }
inline size_t bwd_ws_gr(int64_t M, int64_t D) { return align256(size_t(D) * size_t(gr_cols(M)) * 2); }
inline size_t bwd_ws_part(int64_t M, int64_t D, int64_t N) {
  return bwd_ws_gr(M, D) + align256(size_t(bwd_pg_rows(M, D, N)) * size_t(D) * 4);
}
inline size_t bwd_ws(int64_t M, int64_t D, int64_t N) {
  const KSplit k = dgrad_split(M, D, N);
  return bwd_ws_part(M, D, N) + (k.S > 1 ? align256(size_t(k.S) * size_t(M) * size_t(D) * 4) : 0);
}
// The fused chain backward takes s as side work of its weight-gradient GEMM when each K step's 64 rows
// can be dealt over that GEMM's row tiles at four per block: at least 16 row tiles (D > 3840); with
// fewer, a row kernel computes s. The side work's partials Ps[rowdot_cols(N), M] (one per row and
// 256-column tile) follow the shared backward workspace.
inline bool bwd_rowdot(int64_t D) { return ceil_div(D, kBN) >= 16; }
inline int64_t rowdot_cols(int64_t N) { return ceil_div(N, kBN); }
inline size_t bwd_chain_ws(int64_t M, int64_t D, int64_t N) {
  return bwd_ws(M, D, N) + (bwd_rowdot(D) ? align256(size_t(rowdot_cols(N)) * size_t(M) * 4) : 0);
}
// SwiGLU backward workspace: the fused backward's, then the s partials Ps.
inline size_t bwd_swiglu_ws(int64_t M, int64_t D, int64_t N) {
  return bwd_ws(M, D, N) + align256(size_t(M) * size_t(swiglu_s_cols(N)) * 4);
}
// Unfused SwiGLU backward workspace: the fused backward's, then dO [M, N / 2] bf16.
inline size_t unfused_bwd_swiglu_ws(int64_t M, int64_t D, int64_t N) {
  return bwd_ws(M, D, N) + align256(size_t(M) * size_t(N / 2) * 2);
}

}  // namespace coda

#endif
