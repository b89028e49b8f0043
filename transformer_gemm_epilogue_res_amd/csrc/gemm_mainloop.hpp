// The bf16 MFMA GEMM mainloop shared by every kernel of the chain (gfx950).
//
// Block tile 256 x 256, K step 64, 256 threads = 4 waves in a 2 x 2 grid; each
// wave owns a 128 x 128 sub-tile = 8 x 8 tiles of v_mfma_f32_16x16x32_bf16,
// i.e. 64 fp32x4 accumulators per lane, kept in AGPRs.
//
// Data path:
//   * global -> LDS with buffer_load_dwordx4 ... lds (no VGPR round trip), two
//     64 KB stages; the buffer descriptor is rebased on every K step and its
//     record count is the tensor's remaining bytes, so rows past the end (the
//     ragged last row tile, or a ragged K = M in the weight gradient) read as 0;
//   * LDS -> VGPR: ds_read_b128 for operands whose k is contiguous ("K-rows"
//     tiles), two ds_read_b64_tr_b16 for operands stored MN-major ("K-cols"
//     tiles, e.g. the [in, out] weights), XOR-swizzled layouts so each read hits
//     every one of the 64 banks once per pass.
//
// Schedule of one K step (one wave; the MFMA pipe is the bottleneck, 64 MFMAs
// per 32-wide k slab):
//   slab 0: 64 MFMAs on fragments already in registers, interleaved with the 16
//           DMA loads of the next stage and the 24 LDS reads of slab 1;
//   slab 1: 64 MFMAs; after the first kBarrierAt of them every wave waits for
//           its own DMA and meets the block barrier (the next stage is then
//           complete in LDS and every read of the stage about to be refilled
//           is done), and the remaining MFMAs hide the reads of the next
//           step's slab-0 fragments.
// LDS reads are issued from inline asm with their waits written out (so the
// compiler does not serialise the DMA against them), and scheduling fences
// after every MFMA keep the interleave in program order.
//
// Operand swap: the N-side fragment is the MFMA's src0 and the M-side fragment
// src1, so the 16x16 result tile is C^T and lane l, register e of tile (tm, tn)
// holds C[16 tm + l % 16][16 tn + 4 (l / 16) + e]: four adjacent columns of one
// row (row sums need two cross-lane steps; stores are 8 or 16 bytes).
#ifndef CODA_GEMM_MAINLOOP_HPP
#define CODA_GEMM_MAINLOOP_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "coda_internal.h"

namespace coda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS char lds_char_t;

constexpr int kStageBytes = (kBM + kBN) * kBK * 2;  // 64 KB: A tile then B tile
constexpr int kTileBytes = kBM * kBK * 2;           // 32 KB
constexpr int kSmemBytes = 2 * kStageBytes;
#ifndef CODA_BARRIER_AT
#define CODA_BARRIER_AT 28
#endif
#ifndef CODA_DMA_EVERY
#define CODA_DMA_EVERY 2
#endif
#ifndef CODA_READ_EVERY
#define CODA_READ_EVERY 2
#endif
#ifndef CODA_GROUP_M
#define CODA_GROUP_M 4
#endif
constexpr int kBarrierAt = CODA_BARRIER_AT;  // slab-1 MFMA index of the block barrier
constexpr int kDmaEvery = CODA_DMA_EVERY;    // slab-0 MFMAs per DMA instruction
constexpr int kReadEvery = CODA_READ_EVERY;  // slab-0 MFMAs per LDS read of slab 1

// ------------------------------------------------------------ utilities

template <int... Is, class F>
__device__ __forceinline__ void sfor_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// Calls f(integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices).
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ int64_t dceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ uint32_t lds_u32(const lds_char_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // Raw buffer (stride 0): a lane whose offset is at or past num_records reads 0.
  const int64_t nr = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nr, 0x00020000);
}

// ------------------------------------------------------- LDS tile layouts
//
// K-rows tile: 256 rows (an M or N index) x 64 k, 128 bytes per row (eight
// 16-byte chunks); chunk c of row r is stored at chunk c ^ ((r >> 1) & 7). A
// fragment read (16 consecutive rows, one chunk each) then spans all 64 banks
// per 16-lane pass.
//
// K-cols tile: 64 k-rows x 256 columns, 512 bytes per k-row; chunk c of k-row k
// is stored at c ^ (((k & 3) << 1) | (k & 8)). Each 32-lane pass of a
// transposed fragment read touches k-rows {4j..4j+3} and {8+4j..}, 32 bytes
// each, which this swizzle spreads over all 64 banks.
__device__ __forceinline__ int swz_krows(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_kcols(int k) { return ((k & 3) << 1) | (k & 8); }

// One operand of the GEMM as the mainloop sees it.
//   KROWS: tensor [nrows, ld] with k contiguous; the tile is rows r0 .. r0+255.
//   else : tensor [nk, ld] with the M/N index contiguous; the tile is columns
//          c0 .. c0+255 of k-rows k0 .. k0+63.
template <bool KROWS>
struct Operand {
  const char* base;
  int64_t ld;     // elements
  int64_t extent; // KROWS: nrows; else nk
  int64_t pos0;   // KROWS: r0; else c0
  int64_t K;      // contraction length
  uint32_t voff[8];

  __device__ __forceinline__ void init(const void* b, int64_t ld_, int64_t extent_, int64_t pos0_, int64_t K_,
                                       int wave, int lane) {
    base = static_cast<const char*>(b);
    ld = ld_;
    extent = extent_;
    pos0 = pos0_;
    K = K_;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int seg = q * 4 + wave;  // this wave's q-th 1 KB segment of the 32 KB tile
      if constexpr (KROWS) {
        const int row = seg * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_krows(row);
        voff[q] = uint32_t((int64_t(row) * ld + chunk * 8) * 2);
      } else {
        const int k = seg * 2 + (lane >> 5);
        const int chunk = (lane & 31) ^ swz_kcols(k);
        voff[q] = uint32_t((int64_t(k) * ld + chunk * 8) * 2);
      }
    }
  }

  // Descriptor of K step kt's tile. A K-rows step at or past K gets no records
  // (reads 0); K-rows operands otherwise need K to be a multiple of kBK.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int kt) const {
    const int64_t k0 = int64_t(kt) * kBK;
    if constexpr (KROWS) {
      return make_rsrc(base + (pos0 * ld + k0) * 2, k0 >= K ? 0 : (extent - pos0) * ld * 2 - k0 * 2);
    } else {
      return make_rsrc(base + (k0 * ld + pos0) * 2, (extent - k0) * ld * 2 - pos0 * 2);
    }
  }

  // DMA instruction q (0..7) of this wave into the tile at LDS address dst.
  __device__ __forceinline__ void dma(const __amdgpu_buffer_rsrc_t& rs, lds_char_t* dst, int q, int wave) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (q * 4 + wave) * 1024), 16, voff[q], 0, 0, 0);
  }
};

// Per-lane LDS byte addresses of one operand's fragments (both stages).
//   KROWS: addr[s][kk] for rows wo + l % 16 (tile t adds t * 2048);
//   else : addr[s][t]  for columns wo + 16 t, k-slab 0 low half (slab kk adds
//          kk * 16384, the high half adds 2048).
template <bool KROWS>
struct FragAddr {
  uint32_t addr[2][KROWS ? 2 : 8];
  __device__ __forceinline__ void init(uint32_t tile0, int wo, int lane) {
    const int s = lane & 15, b = lane >> 4;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint32_t tb = tile0 + uint32_t(st * kStageBytes);
      if constexpr (KROWS) {
        const int row = wo + s;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          addr[st][kk] = tb + uint32_t(row * 128 + (((kk * 4 + b) ^ swz_krows(row)) * 16));
      } else {
        const int k = b * 8 + (s >> 2);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int col = wo + 16 * t + 4 * (s & 3);
          addr[st][t] = tb + uint32_t(k * 512 + (((col >> 3) ^ swz_kcols(k)) * 16) + (col & 7) * 2);
        }
      }
    }
  }
};

// A fragment: 8 bf16 (k = 32 kk + 8 (l / 16) + 0..7 of one row or column).
struct Frag {
  bf16x4_t lo, hi;
};

template <int OFF>
__device__ __forceinline__ void ds_read_b128_to(Frag& f, uint32_t addr) {
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  f.lo = __builtin_shufflevector(v, v, 0, 1, 2, 3);
  f.hi = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

template <int OFF>
__device__ __forceinline__ void ds_read_tr_to(bf16x4_t& d, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
}

// The MFMA is inline asm: the "+a" constraint keeps every accumulator in an
// AGPR for the whole loop and the asm order fixes the interleave. The compiler
// therefore knows nothing of its hazards; the ones that can arise are handled
// where they occur: the first k slab writes the accumulators with srcC = 0 (no
// zeroing for the allocator to merge and move), and the mainloop ends with
// padding that the last accumulators pass through (no read of an MFMA result
// before it has landed). check_lds_waits.py verifies this and every LDS wait on
// the generated assembly.
__device__ __forceinline__ void mfma_16x16x32(f32x4_t& c, const Frag& n_side, const Frag& m_side) {
  const bf16x8_t a = __builtin_shufflevector(n_side.lo, n_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b = __builtin_shufflevector(m_side.lo, m_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// The first k slab: c = A B (accumulator input 0), so the accumulators are
// defined by MFMAs alone and no zeroing is ever merged with them.
__device__ __forceinline__ void mfma_16x16x32_first(f32x4_t& c, const Frag& n_side, const Frag& m_side) {
  const bf16x8_t a = __builtin_shufflevector(n_side.lo, n_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b = __builtin_shufflevector(m_side.lo, m_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}

// End of the mainloop: pad past the MFMA result latency; the accumulators of
// the final 16 MFMAs pass through the asm, so no read of them can be placed
// ahead of it.
__device__ __forceinline__ void mfma_drain(f32x4_t (&acc)[8][8]) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3]), "+a"(acc[6][4]),
                 "+a"(acc[6][5]), "+a"(acc[6][6]), "+a"(acc[6][7]), "+a"(acc[7][0]), "+a"(acc[7][1]),
                 "+a"(acc[7][2]), "+a"(acc[7][3]), "+a"(acc[7][4]), "+a"(acc[7][5]), "+a"(acc[7][6]),
                 "+a"(acc[7][7]));
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}

__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Number of LDS instructions that read one fragment.
template <bool KROWS>
constexpr int reads_per_frag() {
  return KROWS ? 1 : 2;
}

// Issue LDS read number R (0 .. 8 * reads_per_frag - 1) of slab KK of stage ST
// for fragment tile R / reads_per_frag into dst[].
template <bool KROWS, int ST, int KK, int R>
__device__ __forceinline__ void frag_read(Frag (&dst)[8], const FragAddr<KROWS>& fa) {
  if constexpr (KROWS) {
    ds_read_b128_to<R * 2048>(dst[R], fa.addr[ST][KK]);
  } else {
    constexpr int t = R / 2;
    if constexpr (R % 2 == 0) ds_read_tr_to<KK * 16384>(dst[t].lo, fa.addr[ST][t]);
    else ds_read_tr_to<KK * 16384 + 2048>(dst[t].hi, fa.addr[ST][t]);
  }
}

// The i-th read of a slab: first the N-side fragments, then the M-side ones.
template <bool A_K, bool B_K, int ST, int KK, int I>
__device__ __forceinline__ void slab_read(Frag (&a)[8], Frag (&b)[8], const FragAddr<A_K>& fa,
                                          const FragAddr<B_K>& fb) {
  constexpr int nb = 8 * reads_per_frag<B_K>();
  if constexpr (I < nb) frag_read<B_K, ST, KK, I>(b, fb);
  else frag_read<A_K, ST, KK, I - nb>(a, fa);
}

template <bool A_K, bool B_K>
constexpr int slab_reads() {
  return 8 * reads_per_frag<A_K>() + 8 * reads_per_frag<B_K>();
}

// Block -> output tile. Consecutive logical tiles go to one XCD (the
// dispatcher deals blocks round-robin over the 8 XCDs); logical tiles are
// rastered down groups of kGroupM tile-rows.
constexpr int kGroupM = CODA_GROUP_M;
__device__ __forceinline__ void map_tile(int64_t M, int64_t N, int& tile_m, int& tile_n) {
  const int tiles_m = int(dceil_div(M, kBM));
  const int tiles_n = int(N / kBN);
  const int nb = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int t = (nb % 8 == 0) ? (b % 8) * (nb / 8) + (b / 8) : b;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int r = t % per_group;
  tile_m = first_m + r % gsz;
  tile_n = r / gsz;
}

struct GemmShape {
  int64_t M, N, K;  // C is M x N, contraction over K
  const void* A;    // A_K: [M, lda] (k contiguous); else [K, lda] (m contiguous)
  int64_t lda;
  const void* B;    // B_K: [N, ldb] (k contiguous); else [K, ldb] (n contiguous)
  int64_t ldb;
};

// One K step on stage ST: see the schedule in the header comment. NEXT says
// whether another K step follows (DMA, barrier and next reads are skipped on
// the last one).
template <bool A_K, bool B_K, int ST, bool NEXT, bool FIRST = false>
__device__ __forceinline__ void kstep(f32x4_t (&acc)[8][8], Frag (&a0)[8], Frag (&b0)[8], Frag (&a1)[8],
                                      Frag (&b1)[8], const FragAddr<A_K>& fa, const FragAddr<B_K>& fb,
                                      const Operand<A_K>& opa, const Operand<B_K>& opb, lds_char_t* smem,
                                      int kt, int wave) {
  constexpr int NR = slab_reads<A_K, B_K>();
  lds_char_t* nxt = smem + (ST ^ 1) * kStageBytes;
  __amdgpu_buffer_rsrc_t ra, rb;
  if constexpr (NEXT) {
    ra = opa.rsrc(kt + 1);
    rb = opb.rsrc(kt + 1);
  }
  // ---- slab 0: MFMAs on (a0, b0) (complete: waited for at the end of the
  // previous step or of the prologue); DMA of the next stage; reads of slab 1
  sfor<64>([&](auto I) {
    constexpr int i = decltype(I)::value;
    if constexpr (FIRST) mfma_16x16x32_first(acc[i / 8][i % 8], b0[i % 8], a0[i / 8]);
    else mfma_16x16x32(acc[i / 8][i % 8], b0[i % 8], a0[i / 8]);
    if constexpr (NEXT && i % kDmaEvery == 0 && i / kDmaEvery < 16) {
      constexpr int q = i / kDmaEvery;  // 0..15: 8 A-tile then 8 B-tile instructions
      if constexpr (q < 8) opa.dma(ra, nxt, q, wave);
      else opb.dma(rb, nxt + kTileBytes, q - 8, wave);
    }
    if constexpr (i % kReadEvery == kReadEvery - 1 && i / kReadEvery < NR)
      slab_read<A_K, B_K, ST, 1, i / kReadEvery>(a1, b1, fa, fb);
  });
  // ---- slab 1: MFMAs on (a1, b1); barrier; reads of the next step's slab 0
  wait_lgkm<0>();
  sfor<64>([&](auto I) {
    constexpr int i = decltype(I)::value;
    mfma_16x16x32(acc[i / 8][i % 8], b1[i % 8], a1[i / 8]);
    if constexpr (NEXT && i == kBarrierAt) wait_vm_barrier();
    if constexpr (NEXT && i > kBarrierAt && i - kBarrierAt - 1 < NR)
      slab_read<A_K, B_K, ST ^ 1, 0, i - kBarrierAt - 1>(a0, b0, fa, fb);
  });
  // the next step's slab-0 fragments (issued 20+ MFMAs ago): nothing stays in
  // flight across the loop back edge or its exit
  wait_lgkm<0>();
}

// acc[tm][tn] (lane l, reg e) = C[m0 + 128 wm + 16 tm + l % 16][n0 + 128 wn + 16 tn + 4 (l / 16) + e]
template <bool A_K, bool B_K>
__device__ __forceinline__ void mainloop(const GemmShape& p, int64_t m0, int64_t n0, lds_char_t* smem,
                                         f32x4_t (&acc)[8][8]) {
  static_assert(slab_reads<A_K, B_K>() <= 64 - kBarrierAt - 1, "slab-0 reads must fit after the barrier");
  static_assert(slab_reads<A_K, B_K>() * kReadEvery <= 64, "slab-1 reads must fit in slab 0");
  static_assert(16 * kDmaEvery <= 64, "the DMA must fit in slab 0");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  Operand<A_K> opa;
  Operand<B_K> opb;
  if constexpr (A_K) opa.init(p.A, p.lda, p.M, m0, p.K, wave, lane);
  else opa.init(p.A, p.lda, p.K, m0, p.K, wave, lane);
  if constexpr (B_K) opb.init(p.B, p.ldb, p.N, n0, p.K, wave, lane);
  else opb.init(p.B, p.ldb, p.K, n0, p.K, wave, lane);
  FragAddr<A_K> fa;
  FragAddr<B_K> fb;
  fa.init(lds_u32(smem), wm * 128, lane);
  fb.init(lds_u32(smem) + kTileBytes, wn * 128, lane);

  // An even number of K steps; a step past K reads zeros (rows past the end of
  // the operand tensors are out of the descriptors' range) and adds nothing.
  const int KT = 2 * int(dceil_div(p.K, 2 * kBK));
  {  // prologue: stage 0 -> LDS, slab-0 fragments -> registers
    const __amdgpu_buffer_rsrc_t ra = opa.rsrc(0), rb = opb.rsrc(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      opa.dma(ra, smem, q, wave);
      opb.dma(rb, smem + kTileBytes, q, wave);
    }
  }
  wait_vm_barrier();
  Frag a0[8], b0[8], a1[8], b1[8];
  sfor<slab_reads<A_K, B_K>()>([&](auto I) { slab_read<A_K, B_K, 0, 0, decltype(I)::value>(a0, b0, fa, fb); });
  wait_lgkm<0>();

  // Every step has the same body: on the last one the "next stage" DMA lies
  // past the end of K (its descriptors have no records, it loads zeros) and the
  // fragments it reads are never used. The first step starts the accumulators.
  kstep<A_K, B_K, 0, true, true>(acc, a0, b0, a1, b1, fa, fb, opa, opb, smem, 0, wave);
  kstep<A_K, B_K, 1, true>(acc, a0, b0, a1, b1, fa, fb, opa, opb, smem, 1, wave);
  for (int kt = 2; kt < KT; kt += 2) {
    kstep<A_K, B_K, 0, true>(acc, a0, b0, a1, b1, fa, fb, opa, opb, smem, kt, wave);
    kstep<A_K, B_K, 1, true>(acc, a0, b0, a1, b1, fa, fb, opa, opb, smem, kt + 1, wave);
  }
  mfma_drain(acc);
}

}  // namespace coda

#endif
