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

// K0, D and N must be multiples of this.
constexpr int64_t kDimQuantum = 256;
// Largest accepted K0 / D / N and M (keeps every per-tile buffer offset < 2^31).
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxRows = int64_t(1) << 24;

// Row block of the unfused RMSNorm-backward kernel (its dgamma partial granularity).
constexpr int kUnfusedBwdRows = 32;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Column count of the forward's sum-of-squares partials P[M, D / kWaveTileN].
inline int64_t ssq_cols(int64_t D) { return D / kWaveTileN; }
// Column count of the SwiGLU backward's s partials Ps[M, (N / 2) / kWaveTileN].
inline int64_t swiglu_s_cols(int64_t N) { return (N / 2) / kWaveTileN; }
// Column count of the cross-entropy tile statistics Pml[M, V / kWaveTileN] (float2).
inline int64_t ce_stat_cols(int64_t V) { return V / kWaveTileN; }
// Cross-entropy forward workspace: Pml, then the target logits [M] fp32.
inline size_t ce_fwd_ws(int64_t M, int64_t V) {
  return align256(size_t(M) * size_t(ce_stat_cols(V)) * 8) + align256(size_t(M) * 4);
}
// Row count of the fused backward's dgamma partials Pg[ceil(M / kWaveTileM), D].
inline int64_t dgamma_rows(int64_t M) { return ceil_div(M, kWaveTileM); }

// Fused backward workspace: bf16(r g) [M, D], then Pg.
inline size_t bwd_ws(int64_t M, int64_t D) {
  return align256(size_t(M) * size_t(D) * 2) + align256(size_t(dgamma_rows(M)) * size_t(D) * 4);
}
// SwiGLU backward workspace: the fused backward's, then the s partials Ps.
inline size_t bwd_swiglu_ws(int64_t M, int64_t D, int64_t N) {
  return bwd_ws(M, D) + align256(size_t(M) * size_t(swiglu_s_cols(N)) * 4);
}
// Unfused SwiGLU backward workspace: the fused backward's, then dO [M, N / 2] bf16.
inline size_t unfused_bwd_swiglu_ws(int64_t M, int64_t D, int64_t N) {
  return bwd_ws(M, D) + align256(size_t(M) * size_t(N / 2) * 2);
}

}  // namespace coda

#endif
