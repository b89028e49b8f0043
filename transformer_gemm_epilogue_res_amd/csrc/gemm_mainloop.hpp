// The bf16 MFMA GEMM mainloop shared by every kernel of the chain (gfx950).
//
// Block tile 256 x 256, K step 64, 512 threads = 8 waves in two groups of 4;
// every SIMD hosts one wave of each group. Group G owns rows 128 G .. 128 G +
// 127 of the block tile and wave p of a group columns 64 p .. 64 p + 63: a
// 128 x 64 sub-tile = 8 x 4 tiles of v_mfma_f32_16x16x32_bf16, i.e. 32 fp32x4
// accumulators per lane, kept in AGPRs.
//
// Ping-pong schedule. The loop runs in phases separated by block barriers; in
// every phase one group multiplies while the other loads:
//
//   phase      0      1      2      3     ...   2 KT-1    2 KT
//   group 0   L(0)   C(0)   L(1)   C(1)   ...   C(KT-1)  (epilogue)
//   group 1    -     L(0)   C(0)   L(1)   ...   L(KT-1)   C(KT-1)
//
// L(k) reads K step k's fragments (both 32-wide k slabs) from LDS into
// registers; C(k) is the wave's 64 MFMAs on them. Each SIMD thus always has
// one wave feeding the MFMA pipe while the other one's LDS reads are in flight,
// and no wave waits on memory while it owns the pipe.
//
// Global -> LDS. The A tiles of the K steps rotate through 3 LDS slots and the
// B tiles through 2 (5 x 32 KB = all 160 KB of a CU's LDS). Group 0 loads the B
// tiles and group 1 the A tiles, each only in its L phases, so no DMA
// instruction ever waits for a memory queue in the middle of an MFMA phase:
//   * B(j+1) is issued at the start of phase 2j (group 0's L(j)) into the slot
//     B(j-1) left, and group 0 waits for it at the end of phase 2j+1;
//   * A(j+2) is issued in phase 2j+1 (group 1's L(j)) into the slot A(j-1)
//     left, and group 1 waits for it at the end of phase 2j+3.
// Each wait precedes a barrier, so a tile is complete in LDS before the phase
// that first reads it, and a slot is refilled only after both groups' reads of
// its previous tile (A(j-1) and B(j-1) are last read in phase 2j-1).
//
// Data path:
//   * global -> LDS with buffer_load_dwordx4 ... lds (no VGPR round trip); the
//     buffer descriptor is rebased on every K step and its
//     record count is the tensor's remaining bytes, so rows past the end (the
//     ragged last row tile, or a ragged K = M in the weight gradient) read as 0;
//   * LDS -> VGPR: ds_read_b128 for operands whose k is contiguous ("K-rows"
//     tiles), two ds_read_b64_tr_b16 for operands stored MN-major ("K-cols"
//     tiles, e.g. the [in, out] weights), XOR-swizzled layouts so each read hits
//     every one of the 64 banks once per pass.
//
// LDS reads, MFMAs, waits and barriers are inline asm, so the compiler can
// neither serialise the DMA against the reads nor move work across phases; it
// also knows none of their hazards, which check_lds_waits.py verifies on the
// generated assembly (LDS waits, MFMA result latency).
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

constexpr int kWaves = kThreads / 64;
constexpr int kTM = kWaveTileM / 16;               // MFMA row tiles per wave
constexpr int kTN = kWaveTileN / 16;               // MFMA column tiles per wave
constexpr int kTileBytes = kBM * kBK * 2;          // 32 KB: one operand tile of one K step
constexpr int kASlots = 3, kBSlots = 2;            // LDS ring slots of the A and B tiles
constexpr int kBBase = kASlots * kTileBytes;       // B slots follow the A slots
constexpr int kSmemBytes = (kASlots + kBSlots) * kTileBytes;  // 160 KB, all of a CU's LDS
constexpr int kEpiWaveBytes = 16384;               // per-wave LDS staging of the epilogue (reuses the slots)
constexpr int kAuxWaveBytes = 4096;                // per-wave LDS of the epilogue's row / column vectors
constexpr int kDmaWaves = 4;                       // one wave group loads each operand
constexpr int kSegs = kTileBytes / 1024 / kDmaWaves;  // 1 KB DMA segments per wave per tile
static_assert(kWaves == 8 && kTM == 8 && kTN == 4, "two groups of four 128 x 64 wave tiles");
static_assert(2 * kWaveTileM == kBM && 4 * kWaveTileN == kBN, "the two groups cover the block tile");
static_assert(kWaves * kEpiWaveBytes <= kSmemBytes, "epilogue staging fits in the slots");

#ifndef CODA_GROUP_M
#define CODA_GROUP_M 4
#endif

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

// One operand of the GEMM as the mainloop sees it, and a loading wave's share
// of its DMA: kSegs of the tile's 32 one-KB segments, segment q * 4 + w for
// wave w of the group that loads this operand.
//   KROWS: tensor [nrows, ld] with k contiguous; the tile is rows r0 .. r0+255;
//          segment s holds rows 8 s .. 8 s + 7.
//   else : tensor [nk, ld] with the M/N index contiguous; the tile is columns
//          c0 .. c0+255 of k-rows k0 .. k0+63; segment s holds k-rows 2 s, 2 s + 1.
// Segment q of a wave lies 32 q rows (8 q k-rows) past segment 0. A K-rows
// segment has the same swizzle for every q; a K-cols segment's swizzle has bit
// 3 = (k & 8) = (q & 1) << 3, so odd and even q keep their own base offset:
// the per-lane byte offset is voff[q & 1] + (q >> 1) * pair_step.
template <bool KROWS>
struct Operand {
  const char* base;
  int64_t ld;     // elements
  int64_t extent; // KROWS: nrows; else nk
  int64_t pos0;   // KROWS: r0; else c0
  int64_t K;      // contraction length
  uint32_t voff[2], pair_step;

  __device__ __forceinline__ void init(const void* b, int64_t ld_, int64_t extent_, int64_t pos0_, int64_t K_,
                                       int wave, int lane) {
    base = static_cast<const char*>(b);
    ld = ld_;
    extent = extent_;
    pos0 = pos0_;
    K = K_;
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      if constexpr (KROWS) {
        const int row = odd * kDmaWaves * 8 + wave * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_krows(row);
        voff[odd] = uint32_t((int64_t(row) * ld + chunk * 8) * 2);
      } else {
        const int k = odd * kDmaWaves * 2 + wave * 2 + (lane >> 5);
        const int chunk = (lane & 31) ^ swz_kcols(k);
        voff[odd] = uint32_t((int64_t(k) * ld + chunk * 8) * 2);
      }
    }
    pair_step = uint32_t((KROWS ? 2 * kDmaWaves * 8 : 2 * kDmaWaves * 2) * ld * 2);
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

  // DMA instruction q (0 .. kSegs-1) of loading wave w into the tile at LDS address dst.
  __device__ __forceinline__ void dma(const __amdgpu_buffer_rsrc_t& rs, lds_char_t* dst, int q, int w) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + (q * kDmaWaves + w) * 1024), 16,
                                             voff[q & 1] + uint32_t(q >> 1) * pair_step, 0, 0, 0);
  }
};

// A fragment: 8 bf16 (k = 32 kk + 8 (l / 16) + 0..7 of one row or column).
struct Frag {
  bf16x4_t lo, hi;
};

// Per-lane LDS byte addresses of one operand's fragments in its first ring
// slot (the others are whole tiles further): NT tiles of 16 rows or columns
// starting at wo (a multiple of 16 NT).
template <bool KROWS, int NT>
struct FragAddr;

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

// K-rows: addr[kk] for row wo + l % 16; tile t adds t * 2048 bytes.
template <int NT>
struct FragAddr<true, NT> {
  uint32_t addr[2];
  __device__ __forceinline__ void init(uint32_t tile0, int wo, int lane) {
    const int s = lane & 15, b = lane >> 4;
    const int row = wo + s;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) addr[kk] = tile0 + uint32_t(row * 128 + (((kk * 4 + b) ^ swz_krows(row)) * 16));
  }
  // Fragment tile T of k slab KK in the stage at byte offset soff.
  template <int KK, int T>
  __device__ __forceinline__ void read(Frag& f, uint32_t soff) const {
    ds_read_b128_to<T * 2048>(f, addr[KK] + soff);
  }
};

// K-cols: lane (s, b) = (l % 16, l / 16) reads k-row k = 8 b + s / 4 (low
// half; the high half is 4 k-rows on, slab 1 is 32 on, both with the same
// swizzle) at column wo + 16 t + 4 (s % 4): chunk wo / 8 + 2 t + (s % 4) / 2,
// byte 8 (s % 2) within it. With W = 2 NT chunks per wave span and wo / 8 a
// multiple of W, the stored chunk is
//   ((wo / 8) ^ (swz & ~(W-1))) + ((2 t) ^ c),  c = (swz & (W-1)) | (s % 4) / 2.
template <int NT>
struct FragAddr<false, NT> {
  uint32_t addr[NT];
  __device__ __forceinline__ void init(uint32_t tile0, int wo, int lane) {
    constexpr int W = 2 * NT;
    const int s = lane & 15, b = lane >> 4;
    const int k = b * 8 + (s >> 2);
    const int swz = swz_kcols(k);
    const int c = (swz & (W - 1)) | ((s & 3) >> 1);
    const uint32_t base = tile0 + uint32_t(k * 512 + ((wo >> 3) ^ (swz & ~(W - 1))) * 16 + (s & 1) * 8);
#pragma unroll
    for (int t = 0; t < NT; ++t) addr[t] = base + uint32_t(((2 * t) ^ c) * 16);
  }
  template <int KK, int T>
  __device__ __forceinline__ void read(Frag& f, uint32_t soff) const {
    const uint32_t a = addr[T] + soff;
    ds_read_tr_to<KK * 16384>(f.lo, a);
    ds_read_tr_to<KK * 16384 + 2048>(f.hi, a);
  }
};

// MFMA as inline asm: "+a" keeps the accumulator in one AGPR for the whole
// loop and the asm order fixes the schedule. The first K step's first slab
// writes the accumulators with srcC = 0 (no zeroing for the allocator to merge
// and move), and the mainloop ends with padding that the last accumulators pass
// through (no read of an MFMA result before it has landed).
template <bool FIRST>
__device__ __forceinline__ void mfma_16x16x32(f32x4_t& c, const Frag& n_side, const Frag& m_side) {
  const bf16x8_t a = __builtin_shufflevector(n_side.lo, n_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b = __builtin_shufflevector(m_side.lo, m_side.hi, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (FIRST) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Pad past the MFMA result latency. The accumulators of the final 16 MFMAs pass
// through the padding asm and all the others through an empty asm after it
// (volatile asm keeps its order), so no read of any accumulator can be placed
// ahead of the padding.
__device__ __forceinline__ void mfma_drain(f32x4_t (&acc)[kTM][kTN]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[4][2]), "+a"(acc[4][3]), "+a"(acc[5][0]),
                 "+a"(acc[5][1]), "+a"(acc[5][2]), "+a"(acc[5][3]), "+a"(acc[6][0]), "+a"(acc[6][1]),
                 "+a"(acc[6][2]), "+a"(acc[6][3]), "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]),
                 "+a"(acc[7][3]));
  asm volatile(""
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                 "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
                 "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
                 "+a"(acc[3][3]));
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Keeps the compiler from moving memory operations across this point (emits nothing).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void prio_high() { asm volatile("s_setprio 1" ::: "memory"); }
__device__ __forceinline__ void prio_low() { asm volatile("s_setprio 0" ::: "memory"); }

// Block -> output tile. Consecutive logical tiles go to one XCD (the
// dispatcher deals blocks round-robin over the 8 XCDs); logical tiles are
// rastered down groups of group_m tile-rows (kGroupM unless the launch names
// another), so at any time an XCD's 32 CUs hold a group_m x (32 / group_m)
// block of tiles.
constexpr int kGroupM = CODA_GROUP_M;
__device__ __forceinline__ void map_tile(int64_t M, int64_t N, int group_m, int& tile_m, int& tile_n) {
  const int tiles_m = int(dceil_div(M, kBM));
  const int tiles_n = int(dceil_div(N, kBN));
  const int nb = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int t = (nb % 8 == 0) ? (b % 8) * (nb / 8) + (b / 8) : b;
  const int gm = group_m > 0 ? group_m : kGroupM;
  const int per_group = gm * tiles_n;
  const int first_m = (t / per_group) * gm;
  const int gsz = min(tiles_m - first_m, gm);
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
  int64_t kslice;   // split-K: block row blockIdx.y contracts k in [y kslice, (y + 1) kslice); 0 = no split
  int group_m = 0;  // tile-rows per raster group (map_tile); 0 = kGroupM
};

// One wave's view of the loop. The A tile of K step s lives in A slot s % 3,
// the B tile in B slot s % 2.
template <bool A_K, bool B_K>
struct Loop {
  Operand<A_K> opa;
  Operand<B_K> opb;
  FragAddr<A_K, kTM> fa;
  FragAddr<B_K, kTN> fb;
  lds_char_t* smem;
  int w4;  // wave index within its group

  // All of this wave's DMA of the A (group 1) or B (group 0) tile of K step s.
  __device__ __forceinline__ void dma_a(int s) const {
    const __amdgpu_buffer_rsrc_t r = opa.rsrc(s);
    lds_char_t* dst = smem + (s % kASlots) * kTileBytes;
#pragma unroll
    for (int q = 0; q < kSegs; ++q) opa.dma(r, dst, q, w4);
  }
  __device__ __forceinline__ void dma_b(int s) const {
    const __amdgpu_buffer_rsrc_t r = opb.rsrc(s);
    lds_char_t* dst = smem + kBBase + (s & 1) * kTileBytes;
#pragma unroll
    for (int q = 0; q < kSegs; ++q) opb.dma(r, dst, q, w4);
  }
  // L(s): this wave's fragments of K step s; N-side first.
  __device__ __forceinline__ void load(int s, Frag (&a)[2][kTM], Frag (&b)[2][kTN]) const {
    const uint32_t sa = uint32_t(s % kASlots) * kTileBytes, sb = uint32_t(s & 1) * kTileBytes;
    sfor<2>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      sfor<kTN>([&](auto T) { fb.template read<kk, decltype(T)::value>(b[kk][T], sb); });
      sfor<kTM>([&](auto T) { fa.template read<kk, decltype(T)::value>(a[kk][T], sa); });
    });
  }
};

// C(k): 64 MFMAs, slab 0 then slab 1, row-tile major, the column tiles in reverse order on odd row
// tiles (serpentine), so that every MFMA of a slab shares one operand fragment with the one before it.
// On this power-limited part fewer operand changes between consecutive MFMAs mean less switching in
// the matrix core: the serpentine order measured about 1 % faster per step than plain row-major.
// The last 16 MFMAs are still those of row tiles 4..7 (what mfma_drain pads). after(I) runs after MFMA I.
template <bool FIRST, class F>
__device__ __forceinline__ void compute(f32x4_t (&acc)[kTM][kTN], const Frag (&a)[2][kTM], const Frag (&b)[2][kTN],
                                        F&& after) {
  sfor<2 * kTM * kTN>([&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr int kk = i / (kTM * kTN), tm = (i / kTN) % kTM;
    constexpr int tn = (tm & 1) ? kTN - 1 - i % kTN : i % kTN;
    mfma_16x16x32<FIRST && kk == 0>(acc[tm][tn], b[kk][tn], a[kk][tm]);
    after(I);
  });
}

// The epilogue's LDS, given K steps KT. Wave 4 G + p gets a 16 KB staging area and 4 KB
// of auxiliary space, all disjoint, placed so that each group may start DMA into them
// during its last K step (the `early` hook of mainloop):
//   group 0 (from the start of its last step, phase 2 KT - 2): the two A slots other
//     than (KT - 1) % 3, which no wave reads again;
//   group 1 (after the barrier that ends phase 2 KT - 1, when both groups' last
//     fragment reads are done): A slot (KT - 1) % 3 and B slot (KT - 1) % 2;
//   auxiliary areas: B slot KT % 2, idle from phase 2 KT - 2 (its last tile, K step
//     KT - 2, was read by phase 2 KT - 3).
__device__ __forceinline__ void epi_regions(lds_char_t* smem, int wave, int KT, lds_char_t*& stage,
                                            lds_char_t*& aux) {
  constexpr int kPerSlot = kTileBytes / kEpiWaveBytes;  // 2 staging areas per slot
  const int sa = (KT - 1) % kASlots, p = wave & 3;
  int region;
  if (wave < 4) {
    const int other = (p >> 1) == 0 ? (sa == 0 ? 1 : 0) : (sa == 2 ? 1 : 2);  // the A slots != sa, ascending
    region = other * kPerSlot + (p & 1);
  } else {
    region = p < 2 ? sa * kPerSlot + p : (kASlots + ((KT - 1) & 1)) * kPerSlot + (p - 2);
  }
  stage = smem + region * kEpiWaveBytes;
  aux = smem + kBBase + (KT & 1) * kTileBytes + wave * kAuxWaveBytes;
}
static_assert(kTileBytes == 2 * kEpiWaveBytes && kWaves * kAuxWaveBytes <= kTileBytes, "epilogue LDS layout");

// Work a kernel may run beside its GEMM, in group 0's phases of the mainloop (group 1 runs the loop
// unchanged). A side with kActive has, per K step k of a group-0 wave:
//   flush(k)     after MFMA 1 of C(k) when k is a positive multiple of kFlush (ahead of the phase's load,
//                so the end-of-phase wait covers its stores): the output of steps k - kFlush .. k - 1;
//                in L(k), ahead of the DMA, it delayed the DMA's issue (the dW1 GEMM measured 7 us slower);
//   read(k)      LDS reads of step k's B tile (slot k % 2) after the L(k) fragment reads, covered by
//                the same LDS wait; landed() follows that wait (asm reads give the compiler no reason
//                to keep their uses behind it);
//   work<I>()    after MFMA I of C(k): the arithmetic on what read(k) and load(k) brought, from I = kAt on;
//   load(k + 1)  right after work<kAt>: one vector-memory load of step k + 1's data into the register
//                work<kAt> has just read (load(0) in the prologue, after B(0)'s DMA).
// The load is then the newest vector-memory operation at the end of C(k), so the wait there for B(k + 1)
// becomes vmcnt(1) and leaves it in flight until C(k + 1); the kernel flushes the last steps after its
// epilogue.
struct NoSide {
  static constexpr bool kActive = false;
};

// Group 0's side of mainloop (below) with a side's work in it.
template <bool A_K, bool B_K, class Early, class Side>
__device__ __forceinline__ void mainloop_side(const Loop<A_K, B_K>& L, int KT, f32x4_t (&acc)[kTM][kTN],
                                              Frag (&a)[2][kTM], Frag (&b)[2][kTN], Early& early, Side& side) {
  L.dma_b(0);
  compiler_fence();  // the side's load is issued after the DMA, as the vmcnt(1) waits assume
  side.load(0);
  wait_vm<1>();  // B(0); the side's load stays in flight
  block_barrier();
  auto step = [&](int k, auto first, auto last) {
    if constexpr (decltype(last)::value) early();
    else L.dma_b(k + 1);
    L.load(k, a, b);
    side.read(k);
    wait_lgkm0();
    side.landed();
    block_barrier();
    prio_high();
    compute<decltype(first)::value>(acc, a, b, [&](auto I) {
      if constexpr (decltype(I)::value == 1) {
        if (k > 0 && k % Side::kFlush == 0) side.flush(k);
      }
      side.template work<decltype(I)::value>();
      if constexpr (decltype(I)::value == Side::kAt && !decltype(last)::value) side.load(k + 1);
    });
    prio_low();
    if constexpr (!decltype(last)::value) wait_vm<1>();  // B(k + 1); the side's load of step k + 1 stays in flight
    block_barrier();
  };
  if (KT == 1) {
    step(0, std::true_type{}, std::true_type{});
  } else {
    step(0, std::true_type{}, std::false_type{});
    for (int k = 1; k < KT - 1; ++k) step(k, std::false_type{}, std::false_type{});
    step(KT - 1, std::false_type{}, std::true_type{});
  }
  mfma_drain(acc);
}

// Group G's side of the loop, for wave 4 G + p:
//   acc[tm][tn] (lane l, reg e) = C[m0 + 128 G + 16 tm + l % 16][n0 + 64 p + 16 tn + 4 (l / 16) + e].
// Both groups pass the same number of barriers (1 + 2 KT). early() issues the
// epilogue's DMA into its LDS (epi_regions) during the last K step: group 0 at the
// start of that step, group 1 after its last barrier; it adds only to vmcnt, which
// the epilogue waits for.
template <bool A_K, bool B_K, int G, class Early, class Side>
__device__ __forceinline__ void mainloop(const GemmShape& p, int64_t m0, int64_t n0, lds_char_t* smem,
                                         f32x4_t (&acc)[kTM][kTN], Early&& early, Side& side) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Loop<A_K, B_K> L;
  L.smem = smem;
  L.w4 = wave & 3;
  if constexpr (A_K) L.opa.init(p.A, p.lda, p.M, m0, p.K, L.w4, lane);
  else L.opa.init(p.A, p.lda, p.K, m0, p.K, L.w4, lane);
  if constexpr (B_K) L.opb.init(p.B, p.ldb, p.N, n0, p.K, L.w4, lane);
  else L.opb.init(p.B, p.ldb, p.K, n0, p.K, L.w4, lane);
  L.fa.init(lds_u32(smem), G * kWaveTileM, lane);
  L.fb.init(lds_u32(smem) + kBBase, L.w4 * kWaveTileN, lane);
  const int KT = int(dceil_div(p.K, kBK));

  Frag a[2][kTM], b[2][kTN];
  if constexpr (Side::kActive && G == 0) {
    mainloop_side(L, KT, acc, a, b, early, side);
    return;
  }
  auto none = [](auto) {};
  // step(k, first, last): the last step is peeled off (its DMA is the epilogue's), so the
  // loop body carries none of it.
  auto run = [&](auto&& step) {
    if (KT == 1) {
      step(0, std::true_type{}, std::true_type{});
    } else {
      step(0, std::true_type{}, std::false_type{});
      for (int k = 1; k < KT - 1; ++k) step(k, std::false_type{}, std::false_type{});
      step(KT - 1, std::false_type{}, std::true_type{});
    }
  };
  if constexpr (G == 0) {
    // prologue: B(0). Phase 2k: the DMA of B(k+1), then L(k); phase 2k+1:
    // C(k), then wait for B(k+1).
    L.dma_b(0);
    wait_vm0();
    block_barrier();
    run([&](int k, auto first, auto last) {
      if constexpr (decltype(last)::value) early();
      else L.dma_b(k + 1);
      L.load(k, a, b);
      wait_lgkm0();
      block_barrier();
      prio_high();
      compute<decltype(first)::value>(acc, a, b, none);
      prio_low();
      if constexpr (!decltype(last)::value) wait_vm0();  // B(k + 1); the last step's DMA is the epilogue's
      block_barrier();
    });
  } else {
    // prologue: A(0), and A(1) left in flight (it is first read in phase 2).
    // Phase 0: nothing; phase 2k+1: the DMA of A(k+2), then L(k), then wait
    // for A(k+1); phase 2k+2: C(k).
    L.dma_a(0);
    if (1 < KT) {
      L.dma_a(1);
      wait_vm<kSegs>();
    } else {
      wait_vm0();
    }
    block_barrier();
    block_barrier();
    run([&](int k, auto first, auto last) {
      const bool more = k + 2 < KT;
      if (more) L.dma_a(k + 2);
      L.load(k, a, b);
      if (more) wait_vm<kSegs>();
      else wait_vm0();
      wait_lgkm0();
      block_barrier();
      if constexpr (decltype(last)::value) early();
      prio_high();
      compute<decltype(first)::value>(acc, a, b, none);
      prio_low();
      if constexpr (!decltype(last)::value) block_barrier();
    });
  }
  mfma_drain(acc);
}

}  // namespace coda

#endif
