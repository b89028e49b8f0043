// HIP kernels for gfx950 (MI355X) and the launching half of the C ABI.
//
// Every GEMM of the chain runs the same MFMA mainloop (gemm_mainloop.hpp); what
// differs is the epilogue that runs on the fp32 accumulator tile while it is
// still in registers (CODA: Rewriting Transformer Blocks as GEMM-Epilogue
// Programs; hotdry blog, section "核心观察": mainloop + epilogue split, and
// section "五类 Epilogue 原语": elementwise maps, vector loads, tile loads and
// stores, tile reductions finished by a light auxiliary kernel).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include "coda.h"
#include "coda_internal.h"
#include "gemm_mainloop.hpp"

namespace coda {

// ----------------------------------------------------------------- helpers

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}

__device__ __forceinline__ void unpack4_bf16(uint2 v, float* o) {
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

__device__ __forceinline__ void unpack8_bf16(uint4 v, float* o) {
  unpack4_bf16(make_uint2(v.x, v.y), o);
  unpack4_bf16(make_uint2(v.z, v.w), o + 4);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Cross-lane reductions of the epilogues on the VALU, with no LDS round trip (shfl_xor is a ds_bpermute):
// * across the four 16-lane rows (the lanes l, l ^ 16, l ^ 32, l ^ 48 that share an output row in the
//   MFMA layout): the gfx950 lane swaps. v_permlane16_swap exchanges the odd rows of its first operand with
//   the even rows of its second, so on two copies of v its two results hold rows (0, 0, 2, 2) and (1, 1, 3, 3),
//   and combining them is v combined with lane l ^ 16; v_permlane32_swap does the same for the two halves
//   (l ^ 32). Sums and maxima are commutative, so every lane gets the bits the xor butterfly gives.
// * within a 16-lane row (the 16 rows of a tile held by one column of lanes): DPP quad permutations for
//   l ^ 1 and l ^ 2, then the row's half-mirror (l <-> 7 - l) and mirror (l <-> 15 - l), which read the
//   same values as l ^ 4 and l ^ 8 once the quads and then the octets are uniform: again the xor
//   butterfly's bits in every lane.
__device__ __forceinline__ float sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_row16(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]: l ^ 1
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]: l ^ 2
  v += dpp_move<0x141>(v);  // row_half_mirror: the other quad of the octet
  v += dpp_move<0x140>(v);  // row_mirror: the other octet of the row
  return v;
}

// e^v as 2^(v log2 e) on the hardware base-2 exponential (one v_exp_f32 after one multiply). Its result is
// within a few fp32 ulps of e^v across the range the epilogues use (the rounding of v log2 e adds a relative
// error of about |v| 2^-24), 0 where e^v underflows and +inf where it overflows -- what the softmax sums and
// the sigmoid want at the ends. Every kernel that must agree bit for bit with another (the recomputing and
// the stored-logits cross-entropy backward, fused and unfused) takes its exponentials from here.
__device__ __forceinline__ float fast_exp(float v) { return __builtin_amdgcn_exp2f(v * 1.4426950408889634f); }

// ------------------------------------------------------ coalesced stores
//
// In the MFMA layout a lane holds four adjacent columns of one row per tile, so
// a direct bf16 store writes 16 rows x 32 bytes per instruction. Instead each
// wave stages its 128 x 64 bf16 block in its own 16 KB of LDS (the mainloop's
// stages are free once the last barrier is passed) and then stores whole
// 128-byte rows, eight lanes x 16 bytes each. The 16-byte chunks of a staged
// row are XOR-swizzled by the row index, so both passes spread over all 64
// banks. fp32 outputs are stored directly (16 bytes per lane).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct StageBf16 {
  lds_char_t* base;
  int lane;
  // Eight bytes of row 16 tm + l % 16 at byte 8 (4 tn + l / 16) of the staged row.
  __device__ __forceinline__ void put_raw(int tm, int tn, u32x2_t p) const {
    const int li = lane & 15, lg = lane >> 4;
    const int row = 16 * tm + li, c = 2 * tn + (lg >> 1);
    *reinterpret_cast<LDS_AS u32x2_t*>(base + row * 128 + ((c ^ (row & 7)) << 4) + (lg & 1) * 8) = p;
  }
  // The four values of tile (tm, tn) of this lane.
  __device__ __forceinline__ void put(int tm, int tn, const f32x4_t& v) const {
    const uint2 p = pack4_bf16(v[0], v[1], v[2], v[3]);
    put_raw(tm, tn, u32x2_t{p.x, p.y});
  }
  // Staged rows to rows mb .. mb+127 (those below M) of out, row stride ldb
  // bytes, starting at byte column cb.
  // NT: non-temporal stores (for an output no kernel reads again soon)
  template <bool NT = false>
  __device__ __forceinline__ void flush_raw(char* out, int64_t ldb, int64_t mb, int64_t cb, int64_t M) const {
    const int c = lane & 7;
#pragma unroll
    for (int q = 0; q < kWaveTileM / 8; ++q) {
      const int row = 8 * q + (lane >> 3);
      const u32x4_t v = *reinterpret_cast<const LDS_AS u32x4_t*>(base + row * 128 + ((c ^ (row & 7)) << 4));
      const int64_t i = mb + row;
      if (i < M) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + i * ldb + cb + 16 * c);
        if constexpr (NT) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
  }
  // Rows mb .. mb+127 (those below M), columns nb .. nb+63 of out[., ldc].
  template <bool NT = false>
  __device__ __forceinline__ void flush(uint16_t* out, int64_t ldc, int64_t mb, int64_t nb, int64_t M) const {
    flush_raw<NT>(reinterpret_cast<char*>(out), 2 * ldc, mb, 2 * nb, M);
  }
  // The reverse of flush: rows mb .. mb+127 (0 past M), columns nb .. nb+63 of src[., ldc] into
  // the staging area with whole-row 16-byte loads; get() then returns a lane's four values.
  __device__ __forceinline__ void fill(const uint16_t* src, int64_t ldc, int64_t mb, int64_t nb, int64_t M) const {
    const int c = lane & 7;
    constexpr int kBatch = kWaveTileM / 16;  // two batches of eight 16-byte loads in flight
#pragma unroll
    for (int q0 = 0; q0 < kWaveTileM / 8; q0 += kBatch) {
      u32x4_t v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int64_t i = mb + 8 * (q0 + q) + (lane >> 3);
        v[q] = i < M ? *reinterpret_cast<const u32x4_t*>(src + i * ldc + nb + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int row = 8 * (q0 + q) + (lane >> 3);
        *reinterpret_cast<LDS_AS u32x4_t*>(base + row * 128 + ((c ^ (row & 7)) << 4)) = v[q];
      }
    }
  }
  // fill()'s staged layout written by LDS DMA: sixteen 1 KB instructions, eight rows each;
  // lane L fills byte slot L % 8 of row L / 8 with global chunk (L % 8) ^ (L / 8). Instruction
  // q gets a descriptor based at row mb + 8 q, so the per-lane offset is the same for all q
  // (and the range check, which covers the lane offset, is exact): rows past M read 0.
  // Completes on vmcnt (wait_vm0 before get()).
  __device__ __forceinline__ void fill_dma(const uint16_t* src, int64_t ldc, int64_t mb, int64_t nb, int64_t M) const {
    const int rl = lane >> 3, c = (lane & 7) ^ rl;
    const uint32_t voff = uint32_t((rl * ldc + 8 * c) * 2);
    const uint16_t* p = src + mb * ldc + nb;
    int64_t bytes = (M - mb) * ldc * 2 - nb * 2;
    lds_char_t* dst = base;
#pragma unroll 1  // one descriptor live at a time (the loop runs inside the mainloop's last step)
    for (int q = 0; q < kWaveTileM / 8; ++q) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p, bytes), (LDS_AS void*)dst, 16, voff, 0, 0, 0);
      p += 8 * ldc;
      bytes -= 16 * ldc;
      dst += 1024;
    }
  }
  // Sixteen bytes (chunk `chunk` of staged row `row`).
  __device__ __forceinline__ u32x4_t get16(int row, int chunk) const {
    return *reinterpret_cast<const LDS_AS u32x4_t*>(base + row * 128 + ((chunk ^ (row & 7)) << 4));
  }
  __device__ __forceinline__ void put16(int row, int chunk, u32x4_t v) const {
    *reinterpret_cast<LDS_AS u32x4_t*>(base + row * 128 + ((chunk ^ (row & 7)) << 4)) = v;
  }
  __device__ __forceinline__ uint2 get(int tm, int tn) const {
    const int li = lane & 15, lg = lane >> 4;
    const int row = 16 * tm + li, c = 2 * tn + (lg >> 1);
    const u32x2_t p = *reinterpret_cast<const LDS_AS u32x2_t*>(base + row * 128 + ((c ^ (row & 7)) << 4) + (lg & 1) * 8);
    return make_uint2(p.x, p.y);
  }
};

// LDS DMA of a vector: the first 256 N bytes at src (0 at or past `bytes`) to dst (wave-uniform),
// 4 bytes per lane and instruction (the bounds check is then exact to the element).
template <int N>
__device__ __forceinline__ void dma_vec(lds_char_t* dst, const void* src, int64_t bytes, int lane) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, bytes);
#pragma unroll
  for (int q = 0; q < N; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + q * 256), 4, uint32_t(q * 256 + lane * 4), 0, 0, 0);
}
__device__ __forceinline__ float lds_f32(const lds_char_t* p) { return *reinterpret_cast<const LDS_AS float*>(p); }
__device__ __forceinline__ int64_t lds_i64(const lds_char_t* p) { return *reinterpret_cast<const LDS_AS int64_t*>(p); }
__device__ __forceinline__ uint2 lds_u2(const lds_char_t* p) {
  const u32x2_t v = *reinterpret_cast<const LDS_AS u32x2_t*>(p);
  return make_uint2(v.x, v.y);
}

// out[rows of tile tm, columns of tile tn] for this lane, fp32 (16 bytes per lane).
__device__ __forceinline__ void store_f32(float* out, int64_t ldc, int64_t mb, int64_t nb, int64_t M, int lane,
                                          int tm, int tn, const f32x4_t& v) {
  const int64_t i = mb + 16 * tm + (lane & 15);
  if (i < M) *reinterpret_cast<float4*>(out + i * ldc + nb + 16 * tn + 4 * (lane >> 4)) = make_float4(v[0], v[1], v[2], v[3]);
}

// Writes the wave's block val(tm, tn) as bf16 (staged) or fp32 (direct).
template <bool F32, bool NT = false, class V>
__device__ __forceinline__ void store_block(lds_char_t* stage, int lane, void* out, int64_t ldc, int64_t mb,
                                            int64_t nb, int64_t M, V&& val) {
  if constexpr (F32) {
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) store_f32(static_cast<float*>(out), ldc, mb, nb, M, lane, tm, tn, val(tm, tn));
  } else {
    const StageBf16 st{stage, lane};
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) st.put(tm, tn, val(tm, tn));
    st.template flush<NT>(static_cast<uint16_t*>(out), ldc, mb, nb, M);
  }
}

// ------------------------------------------------------------ epilogues
// Each epilogue gets the wave's 128 x 64 accumulator block whose first row is
// mb and first column nb, and the wave's LDS staging area. Lane l owns rows
// mb + 16 tm + l % 16 and columns nb + 16 tn + 4 (l / 16) + {0..3}.

// Plain store C = acc (bf16 or fp32).
template <bool F32>
struct EpiStore {
  void* C;
  int64_t ldc, M;
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage) const {
    store_block<F32>(stage, lane, C, ldc, mb, nb, M, [&](int tm, int tn) { return acc[tm][tn]; });
  }
};

// Split-K partial products: block row y writes its fp32 tile to part + y * sstride.
struct EpiPartialF32 {
  float* part;
  int64_t ldc, M, sstride;
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t*) const {
    float* out = part + int64_t(blockIdx.y) * sstride;
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) store_f32(out, ldc, mb, nb, M, lane, tm, tn, acc[tm][tn]);
  }
};

// The weight-gradient GEMM's store, which also finishes dgamma: before its
// mainloop, block b reduces the 64-column chunks b, b + grid, ... of the
// data-gradient GEMM's column partials, dgamma_j = sum_t Pg[t, j], in a fixed
// order (eight row groups t = q mod 8, then the groups in order) -- the
// auxiliary dgamma reduction folded into the kernel that runs next.
template <bool F32>
struct EpiStoreDgamma {
  void* C;
  int64_t ldc, M;
  const float* Pg;
  float* dgamma;
  int64_t rows, D;
  __device__ __forceinline__ void prologue(lds_char_t* smem) const {
    // 64-column chunks dealt round-robin over the blocks (a small GEMM may have fewer blocks than chunks)
    const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
    LDS_AS float* part = reinterpret_cast<LDS_AS float*>(smem);
    for (int64_t chunk = blockIdx.x; chunk < dceil_div(D, 64); chunk += gridDim.x) {  // uniform per block
      const int64_t j = chunk * 64 + c;
      float acc = 0.f;
      if (j < D)
        for (int64_t t = q; t < rows; t += 8) acc += Pg[t * D + j];
      part[q * 64 + c] = acc;
      __syncthreads();
      if (q == 0 && j < D) {
        float tot = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) tot += part[g * 64 + c];
        dgamma[j] = tot;
      }
      __syncthreads();  // part is rewritten by the next chunk; the mainloop's loads overwrite the LDS
    }
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage) const {
    store_block<F32>(stage, lane, C, ldc, mb, nb, M, [&](int tm, int tn) { return acc[tm][tn]; });
  }
};

// The RMSNorm backward's row statistic s_i = sum_n dY_in y_in (hotdry blog, section "反向传播的 GEMM-Epilogue
// 结构": the row dot product of the output gradient with the saved output), as side work of the weight-gradient
// GEMM dW1 = bf16(r g)^T @ dY, which already streams dY: its B tile of K step k holds dY's rows 64 k .. 64 k + 63,
// columns n0 .. n0 + 255 (a K-cols tile). In step k the block of row tile j (of ndt >= 16 row tiles) takes the
// step's rows j + ndt p, p = 0 .. 3, that are below 64 -- every row of every step then has exactly one block
// and slot -- over its 256 columns, wave p of group 0 row slot p: lane l the columns 4 l .. 4 l + 3. Per step a
// lane multiplies the four dY values (read from the B tile with its fragments) by the four y values (loaded one
// step ahead) and adds them (two v_dot2c_f32_bf16); the wave sums the products of each 16-lane row (its 64
// columns) and shifts those sums into a per-row register (lane i of a row: the sum of step k - i), one stage
// after each of six consecutive MFMAs of the step, so that the MFMAs cover the stages' latencies. Every 16
// steps the four rows are added, giving the 16 steps' sums over the tile's 256 columns, which lanes 0 .. 15
// store to Ps[tile_n, i] (i the row). colsum_kernel adds a row's ceil(N / 256) partials in a fixed order.
struct RowDotSide {
  static constexpr bool kActive = true;
  // The arithmetic, and the next step's load after its first stage, start after this MFMA of C(k). At the
  // 8B shape (interleaved runs) 40 .. 52 measured alike, 22 us faster per dW1 GEMM than 8 or 24 (an earlier
  // load finds the memory queue still busy with the phase's DMA) and a little faster than 58.
  static constexpr int kAt = 40;
  static constexpr int kFlush = 16;  // steps per flush: the lanes of one row
  const char* y0;                    // &y[0, n0]
  int64_t ld, rows, tail;            // N, M, bytes of y from y0 on
  float* Ps;                         // this tile's partials: Ps[tile_n, 0 ..]
  uint32_t voff;                     // (row N + 4 l) * 2; past every record when the lane has no row or column
  uint32_t lds;                      // LDS address of the lane's dY values in B slot 0
  int row;                           // the wave's row within a K step, -1 if none
  bool col_ok;
  u32x2_t yv, dv;
  float pv;                          // this step's products, then their 16-lane row sum
  float acc;                         // lane i of each 16-lane row: that row's sum of step k - i

  __device__ __forceinline__ void load(int k) {
    const int64_t k0 = int64_t(k) * kBK;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(y0 + k0 * ld * 2, tail - k0 * ld * 2);
    yv = __builtin_amdgcn_raw_buffer_load_b64(rs, int(voff), 0, 0);
  }
  __device__ __forceinline__ void read(int k) {
    asm volatile("ds_read_b64 %0, %1" : "=v"(dv) : "v"(lds + uint32_t(k & 1) * kTileBytes));
  }
  __device__ __forceinline__ void landed() { asm volatile("" : "+v"(dv)); }
  // After MFMA I of C(k), from I = kAt on, one stage each (an empty volatile asm holds each stage's result
  // there: left alone, the compiler sinks the chain below the last MFMA, onto the phase's critical path):
  // the products, the four adds of the 16-lane row sum, the shift.
  template <int I>
  __device__ __forceinline__ void work() {
    if constexpr (I == kAt) {
      // the halves as scalars first: __builtin_bit_cast of a vector component (dv.y) reads component 0 here
      const uint32_t d0 = dv.x, d1 = dv.y, y0v = yv.x, y1v = yv.y;
      const float v = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_bit_cast(bf16x2_t, d0), __builtin_bit_cast(bf16x2_t, y0v),
          __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, d1), __builtin_bit_cast(bf16x2_t, y1v), 0.f, false),
          false);
      pv = col_ok ? v : 0.f;
    } else if constexpr (I == kAt + 1) {
      pv += dpp_move<0xB1>(pv);   // l ^ 1
    } else if constexpr (I == kAt + 2) {
      pv += dpp_move<0x4E>(pv);   // l ^ 2
    } else if constexpr (I == kAt + 3) {
      pv += dpp_move<0x141>(pv);  // the other quad of the octet
    } else if constexpr (I == kAt + 4) {
      pv += dpp_move<0x140>(pv);  // the other octet: the row's 64 columns, in all its lanes
    } else if constexpr (I == kAt + 5) {
      // acc moves up one lane within each row (DPP row_shr:1); lane 0 of a row, which has no source, keeps pv
      acc = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(pv), __float_as_int(acc), 0x111, 0xF, 0xF, false));
      asm volatile("" : "+v"(acc));
      return;
    }
    if constexpr (I >= kAt && I < kAt + 5) asm volatile("" : "+v"(pv));
  }
  // Steps k0 .. k0 + n - 1 (n <= 16) since the last flush: lane i < n of each row holds step k0 + n - 1 - i.
  __device__ __forceinline__ void flush(int k0, int n) const {
    if (row < 0) return;
    const float tot = sum_rows4(acc);
    const int l = int(__lane_id());
    const int64_t i = (int64_t(k0) + n - 1 - l) * kBK + row;
    if (l < n && i < rows) Ps[i] = tot;
  }
  __device__ __forceinline__ void flush(int k) const { flush(k - kFlush, kFlush); }
};

// The weight-gradient GEMM's plain store of dW1 [D, N], with the row statistic's partials as side work (the
// chain's M rows are this GEMM's contraction; Ps is [ceil(N / 256), M]).
template <bool F32>
struct EpiStoreRowDot {
  void* C;
  int64_t ldc, M;
  const uint16_t* y;
  float* Ps;
  int64_t N, rows;
  int ndt;
  __device__ __forceinline__ RowDotSide side(int tile_m, int tile_n, int64_t n0, int wave, int lane,
                                             lds_char_t* smem) const {
    RowDotSide s;
    const int r = tile_m + ndt * (wave & 3);
    s.row = (wave < 4 && r < kBK) ? r : -1;
    const int col = 4 * lane;
    s.col_ok = n0 + col < N;
    const int rr = s.row < 0 ? 0 : s.row;
    s.voff = (s.row >= 0 && s.col_ok) ? uint32_t((int64_t(rr) * N + col) * 2) : 0x80000000u;
    s.lds = lds_u32(smem) + uint32_t(kBBase + rr * 512 + ((((col >> 3) ^ swz_kcols(rr)) << 4) | ((col & 7) * 2)));
    s.y0 = reinterpret_cast<const char*>(y + n0);
    s.ld = N;
    s.rows = rows;
    s.tail = (rows * N - n0) * 2;
    s.Ps = Ps + int64_t(tile_n) * rows;
    s.yv = s.dv = u32x2_t{0u, 0u};
    s.pv = s.acc = 0.f;
    return s;
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage) const {
    store_block<F32>(stage, lane, C, ldc, mb, nb, M, [&](int tm, int tn) { return acc[tm][tn]; });
  }
};

// GEMM0 epilogue: h = acc + z (fp32) -> store bf16 h; g = bf16(h * gamma) from
// the fp32 h; per-row sum of squares of the fp32 h over the wave's 64 columns,
// left in the wave's auxiliary LDS; after a block barrier finish() adds the four
// waves' sums of each row (in wave order) -> P[i, n0 / 256], the tile's partial.
constexpr int kSsqAuxOffset = 256;  // the 128 row sums follow the 64 gamma values (256 bytes of DMA) in aux
struct EpiResidualSsq {
  const uint16_t* z;
  const uint16_t* gamma;
  uint16_t* h;
  uint16_t* g;
  float* P;
  int64_t M, D, pcols;
  // during the last K step: the z block into the staging area, the wave's 64 gamma values into aux
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t* aux, int64_t mb, int64_t nb, int lane) const {
    StageBf16{stage, lane}.fill_dma(z, D, mb, nb, M);
    dma_vec<1>(aux, gamma + nb, (D - nb) * 2, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t* aux) const {
    const int li = lane & 15, lj = 4 * (lane >> 4);
    wait_vm0();  // early()'s DMA
    float gam[kTN][4];
#pragma unroll
    for (int tn = 0; tn < kTN; ++tn) unpack4_bf16(lds_u2(aux + (16 * tn + lj) * 2), gam[tn]);
    // h = acc + z (z staged by early()) in place, and the row sums of squares
    const StageBf16 zs{stage, lane};
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
      float ssq = 0.f;
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) {
        float zz[4];
        unpack4_bf16(zs.get(tm, tn), zz);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[tm][tn][e] += zz[e];
          ssq += acc[tm][tn][e] * acc[tm][tn][e];
        }
      }
      // the 4 lanes l % 16 == li hold the rest of row i's 64 columns
      ssq = sum_rows4(ssq);
      if (lane < 16) *reinterpret_cast<LDS_AS float*>(aux + kSsqAuxOffset + (16 * tm + li) * 4) = ssq;
    }
    store_block<false>(stage, lane, h, D, mb, nb, M, [&](int tm, int tn) { return acc[tm][tn]; });
    store_block<false>(stage, lane, g, D, mb, nb, M, [&](int tm, int tn) {
      f32x4_t v = acc[tm][tn];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= gam[tn][e];
      return v;
    });
  }
  // After the block barrier, all waves: wave p of a group adds rows 32 p .. 32 p + 31 of its group's
  // 128 (first row mb) over the group's waves whose columns lie below D (aux0: the group's first wave's
  // auxiliary area) and writes P[i, n0 / 256].
  __device__ __forceinline__ void finish(const lds_char_t* aux0, int64_t mb, int64_t n0, int p, int lane) const {
    const int64_t left = (D - n0) / kWaveTileN;
    const int nvalid = left < 4 ? int(left) : 4;
    if (lane < 32) {
      const int row = 32 * p + lane;
      float s = lds_f32(aux0 + kSsqAuxOffset + row * 4);
      for (int w = 1; w < nvalid; ++w) s += lds_f32(aux0 + w * kAuxWaveBytes + kSsqAuxOffset + row * 4);
      const int64_t i = mb + row;
      if (i < M) P[i * pcols + n0 / kBN] = s;
    }
  }
};

// The row scales of GEMM1's epilogues, r_i = 1 / sqrt(sum_t P[i, t] / D + eps) (the deferred RMSNorm
// factor). FOLD: each wave combines them itself from the sums of squares P [M, pcols] of its 128 rows,
// brought into its staging area by DMA during the last K step (and read before the staging area is
// reused): the four lanes of a row each add a strided share of its partials, then two butterfly steps
// add the shares -- a fixed order that depends only on pcols, so every tile of a row gets the same
// bits -- and the waves of tile column 0 write r. Otherwise (a separate kernel combined them) r is an
// input, moved into aux. The two are separate instantiations, so neither carries the other's registers.
template <bool FOLD>
struct RowScaleSrc {
  float* r;
  const float* P;  // FOLD only
  int64_t M, pcols;
  float D, eps;
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t* aux, int64_t mb, int lane) const {
    if constexpr (!FOLD) {
      dma_vec<2>(aux, r + mb, (M - mb) * 4, lane);
    } else {
      // rows mb .. mb + 127 of P: 512 pcols contiguous bytes (0 past row M - 1)
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(P + mb * pcols, (M - mb) * pcols * 4);
      if ((pcols & 3) == 0) {  // 16 bytes per lane: the rows are 16-byte multiples, so no chunk straddles row M
#pragma unroll 1
        for (int q = 0; q < pcols / 2; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(stage + q * 1024), 16, uint32_t(q * 1024 + lane * 16), 0, 0, 0);
      } else {  // 4 bytes per lane (exact to the element)
#pragma unroll 1
        for (int q = 0; q < 2 * pcols; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(stage + q * 256), 4, uint32_t(q * 256 + lane * 4), 0, 0, 0);
      }
    }
  }
  // rr[tm]: the scale of row mb + 16 tm + l % 16 (after early()'s DMA has landed)
  __device__ __forceinline__ void scales(float (&rr)[kTM], const lds_char_t* stage, const lds_char_t* aux, int64_t mb,
                                         int64_t nb, int lane) const {
    const int li = lane & 15, lg = lane >> 4;
    if constexpr (!FOLD) {
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm) rr[tm] = lds_f32(aux + (16 * tm + li) * 4);
    } else {
      const int pc = int(pcols);  // at most 32 partials: 32-bit LDS offsets
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm) {
        const int row = 16 * tm + li;
        float s = 0.f;
        for (int q = lg; q < pc; q += 4) s += lds_f32(stage + (row * pc + q) * 4);
        s = sum_rows4(s);
        rr[tm] = 1.0f / sqrtf(s / D + eps);
      }
      if (nb == 0 && lg == 0) {
#pragma unroll
        for (int tm = 0; tm < kTM; ++tm) {
          const int64_t i = mb + 16 * tm + li;
          if (i < M) r[i] = rr[tm];
        }
      }
    }
  }
};
static_assert(kWaveTileM * 4 * kFoldedCombineMaxCols <= kEpiWaveBytes, "a wave's partials fit its staging area");

// GEMM1 epilogue: y = r_i * acc (the deferred RMSNorm row scale).
template <bool F32, bool FOLD>
struct EpiRowScale {
  RowScaleSrc<FOLD> rs;
  void* y;
  int64_t N;
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t* aux, int64_t mb, int64_t, int lane) const {
    rs.early(stage, aux, mb, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t* aux) const {
    wait_vm0();
    float rr[kTM];
    rs.scales(rr, stage, aux, mb, nb, lane);
    // y non-temporally: the forward does not read it again and the backward reads it once (the dW1 GEMM's
    // side work, or the row-statistic kernel, which this made about 30 us faster at the 8B shape)
    store_block<F32, true>(stage, lane, y, N, mb, nb, rs.M, [&](int tm, int tn) {
      f32x4_t v = acc[tm][tn];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= rr[tm];
      return v;
    });
  }
};

// ---------------------------------------------------------------- SwiGLU
// Column 2f of y is gate f and 2f+1 up f (blog, section "成对激活的寄存器级融合":
// paired features in adjacent output columns). In the MFMA layout a lane holds
// four adjacent columns 16 tn + 4 (l / 16) + {0..3} of a row, i.e. two whole
// pairs, so the activation and its backward are lane-local.

// sigma(v) = 1 / (1 + e^-v) with the hardware reciprocal (v_rcp_f32, about 1 ulp): 0 as v -> -inf (1 / inf),
// 1 as v -> +inf, NaN for NaN.
__device__ __forceinline__ float sigmoidf_(float v) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-v)); }

// Staging of a 128 x 32 bf16 block (64-byte rows; 16-byte chunk c of row r at
// c ^ ((r >> 2) & 3), which spreads both passes over all 64 banks). put() takes
// the two values of columns 8 tn + 2 (l / 16) + {0, 1} of row 16 tm + l % 16.
struct StageBf16Half {
  lds_char_t* base;
  int lane;
  __device__ __forceinline__ void put(int tm, int tn, float a, float b) const {
    const int li = lane & 15, lg = lane >> 4;
    const int row = 16 * tm + li;
    *reinterpret_cast<LDS_AS uint32_t*>(base + row * 64 + ((tn ^ ((row >> 2) & 3)) << 4) + 4 * lg) = pack2_bf16(a, b);
  }
  __device__ __forceinline__ void flush(uint16_t* out, int64_t ldc, int64_t mb, int64_t nb, int64_t M) const {
    const int c = lane & 3;
#pragma unroll
    for (int q = 0; q < kWaveTileM / 16; ++q) {
      const int row = 16 * q + (lane >> 2);
      const u32x4_t v = *reinterpret_cast<const LDS_AS u32x4_t*>(base + row * 64 + ((c ^ ((row >> 2) & 3)) << 4));
      const int64_t i = mb + row;
      if (i < M) *reinterpret_cast<u32x4_t*>(out + i * ldc + nb + 8 * c) = v;
    }
  }
};

// GEMM1 epilogue with SwiGLU: y = r_i * acc (stored in bf16: the backward needs
// the gate and up values) and o_if = silu(y_i,2f) * y_i,2f+1 from the fp32 y,
// stored in fp32 (F32) or bf16.
template <bool F32, bool FOLD>
struct EpiRowScaleSwiglu {
  RowScaleSrc<FOLD> rs;
  void* y;
  void* o;
  int64_t N;  // o has N / 2 columns
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t* aux, int64_t mb, int64_t, int lane) const {
    rs.early(stage, aux, mb, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t* aux) const {
    const int64_t M = rs.M;
    wait_vm0();
    float rr[kTM];
    rs.scales(rr, stage, aux, mb, nb, lane);
    store_block<false>(stage, lane, y, N, mb, nb, M, [&](int tm, int tn) {
      f32x4_t v = acc[tm][tn];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= rr[tm];
      return v;
    });
    const int64_t F = N / 2, ob = nb / 2;  // the wave's 32 columns of o start at nb / 2
    const StageBf16Half st{stage, lane};
    const StageBf16 sf{stage, lane};
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = rr[tm] * acc[tm][tn][e];
        const float o0 = v[0] * sigmoidf_(v[0]) * v[1], o1 = v[2] * sigmoidf_(v[2]) * v[3];
        if constexpr (F32) sf.put_raw(tm, tn, u32x2_t{__float_as_uint(o0), __float_as_uint(o1)});
        else st.put(tm, tn, o0, o1);
      }
    }
    // the wave's 128 x 32 block of o: fp32 rows are 128 bytes, as the bf16 y rows
    if constexpr (F32) sf.flush_raw(static_cast<char*>(o), 4 * F, mb, 4 * ob, M);
    else st.flush(static_cast<uint16_t*>(o), F, mb, ob, M);
  }
};

// Staging of 64 rows x 256 bytes (a wave's y or dY block for 4 of its 8 row
// tiles): 16-byte chunk c of row r at c ^ (r & 15), so 16 lanes reading one
// chunk of 16 consecutive rows, and 16 lanes reading one whole row, each touch
// all 64 banks once.
struct StageRows256 {
  lds_char_t* base;
  int lane;
  __device__ __forceinline__ int off(int row, int chunk) const { return row * 256 + ((chunk ^ (row & 15)) << 4); }
  // rows mb .. mb+63 (0 past M), 128 bf16 columns from cb, of src[., ldc]
  __device__ __forceinline__ void fill(const uint16_t* src, int64_t ldc, int64_t mb, int64_t cb, int64_t M) const {
    const int c = lane & 15;
#pragma unroll
    for (int q0 = 0; q0 < 16; q0 += 8) {
      u32x4_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t i = mb + 4 * (q0 + q) + (lane >> 4);
        v[q] = i < M ? *reinterpret_cast<const u32x4_t*>(src + i * ldc + cb + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        *reinterpret_cast<LDS_AS u32x4_t*>(base + off(4 * (q0 + q) + (lane >> 4), c)) = v[q];
    }
  }
  __device__ __forceinline__ void flush(uint16_t* out, int64_t ldc, int64_t mb, int64_t cb, int64_t M) const {
    const int c = lane & 15;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 4 * q + (lane >> 4);
      const u32x4_t v = *reinterpret_cast<const LDS_AS u32x4_t*>(base + off(row, c));
      const int64_t i = mb + row;
      if (i < M) *reinterpret_cast<u32x4_t*>(out + i * ldc + cb + 8 * c) = v;
    }
  }
  // fill()'s staged layout written by LDS DMA: sixteen 1 KB instructions of four rows each; lane L fills
  // 16-byte slot L % 16 of row 4 q + L / 16 with global chunk (L % 16) ^ (row & 15). Instruction q's
  // descriptor is based at row mb + 4 q, so the range check (which covers the lane offset) is exact:
  // rows past M read 0. Completes on vmcnt (wait_vm0 before get()).
  __device__ __forceinline__ void fill_dma(const uint16_t* src, int64_t ldc, int64_t mb, int64_t cb, int64_t M) const {
    const int rl = lane >> 4;
    const uint16_t* p = src + mb * ldc + cb;
    int64_t bytes = (M - mb) * ldc * 2 - cb * 2;
    lds_char_t* dst = base;
#pragma unroll 1  // one descriptor live at a time (the loop runs inside the mainloop's last step)
    for (int q = 0; q < 16; ++q) {
      const int c = (lane & 15) ^ ((4 * q + rl) & 15);
      const uint32_t voff = uint32_t((rl * ldc + 8 * c) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p, bytes), (LDS_AS void*)dst, 16, voff, 0, 0, 0);
      p += 4 * ldc;
      bytes -= 8 * ldc;
      dst += 1024;
    }
  }
  __device__ __forceinline__ u32x4_t get(int row, int chunk) const {
    return *reinterpret_cast<const LDS_AS u32x4_t*>(base + off(row, chunk));
  }
  __device__ __forceinline__ void put(int row, int chunk, u32x4_t v) const {
    *reinterpret_cast<LDS_AS u32x4_t*>(base + off(row, chunk)) = v;
  }
};

// Epilogue of the output projection's data gradient dO = dOut @ W2^T with the
// SwiGLU backward (the dimension-expanding step): for the four features
// f = nb + 16 tn + 4 (l / 16) + {0..3} of a lane it takes the saved gate/up pairs
// y[i, 2f], y[i, 2f+1], writes
//   dY[i, 2f] = dO up silu'(gate),  dY[i, 2f+1] = dO silu(gate)   (bf16)
// and the row statistic's partial sum over the wave's 64 features,
//   Ps[i, nb / 64] = sum over its 128 columns of dY y   (fp32 dY, bf16 y).
// The wave's 128 x 128 block of y passes through the staging area in two halves
// of 64 rows, read and written as whole 256-byte rows; each lane's dY replaces
// the y it has just read, and the half is then stored. The first half is moved in
// by DMA during the last K step, the second after the first has been stored.
struct EpiSwigluBwd {
  const uint16_t* y;
  uint16_t* dY;
  float* Ps;
  int64_t M, F, pcols;
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t*, int64_t mb, int64_t nb, int lane) const {
    StageRows256{stage, lane}.fill_dma(y, 2 * F, mb, 2 * nb, M);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t*) const {
    const int li = lane & 15, lg = lane >> 4;
    const StageRows256 st{stage, lane};
    wait_vm0();  // early()'s DMA of the first half
    auto do_half = [&](auto H) {  // H: std::integral_constant, so every acc index is a constant
      constexpr int half = decltype(H)::value;
      const int64_t hb = mb + 64 * half;  // first row of this half
      if constexpr (half == 1) st.fill(y, 2 * F, hb, 2 * nb, M);
#pragma unroll
      for (int t = 0; t < kTM / 2; ++t) {
        const int tm = (kTM / 2) * half + t, row = 16 * t + li;
        float part = 0.f;
#pragma unroll
        for (int tn = 0; tn < kTN; ++tn) {
          const int chunk = 4 * tn + lg;
          const u32x4_t raw = st.get(row, chunk);
          float yv[8], d[8];
          unpack8_bf16(make_uint4(raw.x, raw.y, raw.z, raw.w), yv);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gate = yv[2 * e], up = yv[2 * e + 1], dO = acc[tm][tn][e];
            const float sg = sigmoidf_(gate);
            d[2 * e] = dO * up * (sg * (1.0f + gate * (1.0f - sg)));
            d[2 * e + 1] = dO * (gate * sg);
            part += d[2 * e] * gate + d[2 * e + 1] * up;
          }
          const uint2 lo = pack4_bf16(d[0], d[1], d[2], d[3]), hi = pack4_bf16(d[4], d[5], d[6], d[7]);
          st.put(row, chunk, u32x4_t{lo.x, lo.y, hi.x, hi.y});
        }
        // the 4 lanes l % 16 == li hold the rest of row i's 64 features
        part = sum_rows4(part);
        const int64_t i = hb + row;
        if (lane < 16 && i < M) Ps[i * pcols + nb / kWaveTileN] = part;
      }
      st.flush(dY, 2 * F, hb, 2 * nb, M);
    };
    do_half(std::integral_constant<int, 0>{});
    do_half(std::integral_constant<int, 1>{});
  }
};

// ---------------------------------------------------------- cross-entropy
// LM-head GEMM logits = h @ W^T with the stateful log-sum-exp epilogue (blog,
// section "五类 Epilogue 原语": tile-level online log-sum-exp / cross-entropy
// statistics). A target outside [0, V) marks an ignored row.

__device__ __forceinline__ bool ce_valid(int64_t t, int64_t V) { return t >= 0 && t < V; }

// Per (row, wave tile of 64 columns): the running statistics of the row's
// logits over those columns, m = max and l = sum exp(logit - m) -> Pml[i, nb / 64];
// the lane that holds column t_i writes the target logit to tgt[i]. STORE: the fp32
// logits are also written to logits[M, V].
template <bool STORE>
struct EpiCeStats {
  const int64_t* targets;
  float2* Pml;
  float* tgt;
  float* logits;
  int64_t M, V, pcols;
  // during the last K step: the wave's 128 targets into aux
  __device__ __forceinline__ void early(lds_char_t*, lds_char_t* aux, int64_t mb, int64_t, int lane) const {
    dma_vec<4>(aux, targets + mb, (M - mb) * 8, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t*, lds_char_t* aux) const {
    const int li = lane & 15, lg = lane >> 4;
    wait_vm0();  // early()'s DMA (before any store: vmcnt counts stores too)
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
      const int64_t i = mb + 16 * tm + li;
      const bool ok = i < M;
      float m = -INFINITY;
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, acc[tm][tn][e]);
      m = max_rows4(m);
      float l = 0.f;
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn)
#pragma unroll
        for (int e = 0; e < 4; ++e) l += fast_exp(acc[tm][tn][e] - m);
      l = sum_rows4(l);
      if (ok && lg == 0) Pml[i * pcols + nb / kWaveTileN] = make_float2(m, l);
      const int64_t t = ok ? lds_i64(aux + (16 * tm + li) * 8) : -1;
      const int64_t c = t - nb;  // the target's column inside the wave tile
      if (ok && ce_valid(t, V) && c >= 0 && c < kWaveTileN && ((c >> 2) & 3) == lg) {
        float v = 0.f;
#pragma unroll
        for (int tn = 0; tn < kTN; ++tn)
#pragma unroll
          for (int e = 0; e < 4; ++e) v = (16 * tn + 4 * lg + e == c) ? acc[tm][tn][e] : v;
        tgt[i] = v;
      }
    }
    if constexpr (STORE) {  // after the statistics (issued first they make the compiler spill)
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < kTN; ++tn) store_f32(logits, V, mb, nb, M, lane, tm, tn, acc[tm][tn]);
    }
  }
};

// Backward epilogue on the recomputed logits: dlogits = dloss_i (exp(logit - lse_i)
// - [v = t_i]), 0 on ignored rows; stored bf16 (the operand of the two GEMMs that follow).
struct EpiCeBwd {
  const int64_t* targets;
  const float* lse;
  const float* dloss;
  uint16_t* dlogits;
  int64_t M, V;
  // during the last K step: the wave's 128 targets, lse and dloss values into aux
  __device__ __forceinline__ void early(lds_char_t*, lds_char_t* aux, int64_t mb, int64_t, int lane) const {
    dma_vec<4>(aux, targets + mb, (M - mb) * 8, lane);
    dma_vec<2>(aux + 1024, lse + mb, (M - mb) * 4, lane);
    dma_vec<2>(aux + 2048, dloss + mb, (M - mb) * 4, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t* aux) const {
    const int li = lane & 15, lg = lane >> 4;
    wait_vm0();
    float ls[kTM], dl[kTM];
    int tc[kTM];
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
      const int row = 16 * tm + li;
      const int64_t i = mb + row;
      const int64_t t = i < M ? lds_i64(aux + row * 8) : -1;
      const bool ok = i < M && ce_valid(t, V);
      // an ignored row takes lse = +inf, so exp() is 0 there rather than overflowing to inf
      // (0 * inf would make its zero gradient NaN)
      ls[tm] = ok ? lds_f32(aux + 1024 + row * 4) : INFINITY;
      dl[tm] = ok ? lds_f32(aux + 2048 + row * 4) : 0.f;
      const int64_t c = t - nb - 4 * lg;  // target column relative to the lane's first column of tile 0
      tc[tm] = (c >= 0 && c < kWaveTileN) ? int(c) : -1;
    }
    store_block<false>(stage, lane, dlogits, V, mb, nb, M, [&](int tm, int tn) {
      f32x4_t d;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp(acc[tm][tn][e] - ls[tm]);
        d[e] = dl[tm] * (p - (tc[tm] == 16 * tn + e ? 1.0f : 0.0f));
      }
      return d;
    });
  }
};

// Data-gradient epilogue on G = dY @ W1^T:
//   da = r gamma G - (s r^2 / D) h,  Pg[row tile, j] = sum over the wave's 128 rows of G r h.
template <bool F32>
struct EpiRmsNormBwd {
  const uint16_t* h;
  const float* r;
  const float* s;
  const uint16_t* gamma;
  void* da;
  float* Pg;
  int64_t M, D;
  // during the last K step: the h block into the staging area; r, s (0 past M) and the wave's 64
  // gamma values into aux
  __device__ __forceinline__ void early(lds_char_t* stage, lds_char_t* aux, int64_t mb, int64_t nb, int lane) const {
    StageBf16{stage, lane}.fill_dma(h, D, mb, nb, M);
    dma_vec<2>(aux, r + mb, (M - mb) * 4, lane);
    dma_vec<2>(aux + 1024, s + mb, (M - mb) * 4, lane);
    dma_vec<1>(aux + 2048, gamma + nb, (D - nb) * 2, lane);
  }
  __device__ __forceinline__ void operator()(f32x4_t (&acc)[kTM][kTN], int64_t mb, int64_t nb, int lane,
                                             lds_char_t* stage, lds_char_t* aux) const {
    const int li = lane & 15, lj = 4 * (lane >> 4);
    const float invD = 1.0f / float(D);
    wait_vm0();  // early()'s DMA
    // each lane's bf16 da for a (tm, tn) tile takes the place of the h values it has just read
    const StageBf16 st{stage, lane};
    float rr[kTM], c2[kTM];
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) {
      const int row = 16 * tm + li;
      rr[tm] = lds_f32(aux + row * 4);
      c2[tm] = lds_f32(aux + 1024 + row * 4) * rr[tm] * rr[tm] * invD;
    }
    // da tile by tile, and the dgamma column partials
#pragma unroll
    for (int tn = 0; tn < kTN; ++tn) {
      const int64_t j = nb + 16 * tn + lj;
      float gam[4], cs[4] = {0.f, 0.f, 0.f, 0.f};
      unpack4_bf16(lds_u2(aux + 2048 + (16 * tn + lj) * 2), gam);
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm) {
        float hv[4];
        unpack4_bf16(st.get(tm, tn), hv);
        f32x4_t d;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float G = acc[tm][tn][e];
          cs[e] += G * rr[tm] * hv[e];
          d[e] = rr[tm] * gam[e] * G - c2[tm] * hv[e];
        }
        if constexpr (F32) store_f32(static_cast<float*>(da), D, mb, nb, M, lane, tm, tn, d);
        else st.put(tm, tn, d);
      }
      // column sums over the 16 lanes sharing l / 16 (they hold the 16 rows of each tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cs[e] = sum_row16(cs[e]);
      }
      if (li == 0 && mb < M)  // a wave whose rows all lie past M has no Pg row
        *reinterpret_cast<float4*>(Pg + (mb / kWaveTileM) * D + j) = make_float4(cs[0], cs[1], cs[2], cs[3]);
    }
    if constexpr (!F32) st.flush(static_cast<uint16_t*>(da), D, mb, nb, M);
  }
};

// An epilogue may also carry block-level work that runs before the mainloop
// (prologue(smem), all threads; the LDS is free until the mainloop starts).
template <class Epi, class = void>
struct HasPrologue : std::false_type {};
template <class Epi>
struct HasPrologue<Epi, decltype(std::declval<const Epi&>().prologue(nullptr), void())> : std::true_type {};
// ... and DMA of its inputs into its LDS during the last K step (early(stage, aux, mb, nb,
// lane)); such an epilogue takes the auxiliary area too and waits for that DMA itself.
template <class Epi, class = void>
struct HasEarly : std::false_type {};
template <class Epi>
struct HasEarly<Epi, decltype(std::declval<const Epi&>().early(nullptr, nullptr, 0, 0, 0), void())> : std::true_type {};

// ... and block-level work after the epilogue (finish(aux0, mb, n0, p, lane), every wave, after a block
// barrier that every wave reaches, including waves whose columns lie past N; aux0 is the auxiliary
// area of the wave's group's first wave, mb the group's first row, p the wave's index in the group).
template <class Epi, class = void>
struct HasFinish : std::false_type {};
template <class Epi>
struct HasFinish<Epi, decltype(std::declval<const Epi&>().finish(nullptr, 0, 0, 0, 0), void())> : std::true_type {};

// ... and side work in the mainloop (side(tile_m, tile_n, n0, wave, lane, smem) gives the wave's side
// object, see NoSide); such a GEMM is never split over its contraction.
template <class Epi, class = void>
struct HasSide : std::false_type {};
template <class Epi>
struct HasSide<Epi, decltype(std::declval<const Epi&>().side(0, 0, 0, 0, 0, nullptr), void())> : std::true_type {};
template <class Epi>
__device__ __forceinline__ auto make_side(const Epi& epi, int tile_m, int tile_n, int64_t n0, int wave, int lane,
                                          lds_char_t* smem) {
  if constexpr (HasSide<Epi>::value) return epi.side(tile_m, tile_n, n0, wave, lane, smem);
  else return NoSide{};
}

template <bool A_K, bool B_K, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmShape p0, const Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kSmemBytes];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  if constexpr (HasPrologue<Epi>::value) epi.prologue(smem);
  GemmShape p = p0;
  if (p0.kslice > 0) {  // split-K: this block row's slice of the contraction (k offset along the k-contiguous dim or the rows)
    const int64_t k0 = int64_t(blockIdx.y) * p0.kslice;
    p.K = p0.K - k0 < p0.kslice ? p0.K - k0 : p0.kslice;
    p.A = static_cast<const char*>(p0.A) + 2 * (A_K ? k0 : k0 * p0.lda);
    p.B = static_cast<const char*>(p0.B) + 2 * (B_K ? k0 : k0 * p0.ldb);
  }
  int tile_m, tile_n;
  map_tile(p.M, p.N, p.group_m, tile_m, tile_n);
  const int64_t m0 = int64_t(tile_m) * kBM, n0 = int64_t(tile_n) * kBN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t nb = n0 + (wave & 3) * kWaveTileN;
  lds_char_t *stage, *aux;
  epi_regions(smem, wave, int(dceil_div(p.K, kBK)), stage, aux);
  f32x4_t acc[kTM][kTN];
  // N is a multiple of the wave tile width (64), so a wave's columns lie wholly inside or wholly past
  // N: in the last column tile, a wave past N runs the mainloop (its loads read zeros or other rows'
  // values, in bounds) but writes nothing -- no output, no partial statistics.
  const bool cols_in = nb < p.N;
  auto side = make_side(epi, tile_m, tile_n, n0, wave, lane, smem);
  if (wave < 4) {
    mainloop<A_K, B_K, 0>(p, m0, n0, smem, acc, [&] {
      if constexpr (HasEarly<Epi>::value) epi.early(stage, aux, m0, nb, lane);
    }, side);
    if (!cols_in) {
      wait_vm0();
    } else if constexpr (HasEarly<Epi>::value) {
      epi(acc, m0, nb, lane, stage, aux);
    } else {
      epi(acc, m0, nb, lane, stage);
    }
  } else {
    mainloop<A_K, B_K, 1>(p, m0, n0, smem, acc, [&] {
      if constexpr (HasEarly<Epi>::value) epi.early(stage, aux, m0 + kWaveTileM, nb, lane);
    }, side);
    if (!cols_in) {
      wait_vm0();
    } else if constexpr (HasEarly<Epi>::value) {
      epi(acc, m0 + kWaveTileM, nb, lane, stage, aux);
    } else {
      epi(acc, m0 + kWaveTileM, nb, lane, stage);
    }
  }
  if constexpr (decltype(side)::kActive) {  // the steps since the loop's last flush
    const int KT = int(dceil_div(p.K, kBK)), F = decltype(side)::kFlush;
    side.flush((KT - 1) / F * F, (KT - 1) % F + 1);
  }
  if constexpr (HasFinish<Epi>::value) {
    wait_lgkm0();  // this wave's LDS writes for finish()
    block_barrier();
    epi.finish(aux - (wave & 3) * kAuxWaveBytes, m0 + (wave >> 2) * kWaveTileM, n0, wave & 3, lane);
  }
}

// ------------------------------------------------------- small kernels

// r_i = 1 / sqrt(sum_t P[i, t] / D + eps). Sixteen lanes per row, each summing
// a strided share of the row's partials (as float4 loads when the rows are
// 16-byte aligned), then a fixed butterfly over the 16 lanes: the summation
// order depends only on pcols.
constexpr int kCombineRows = 16;  // rows per 256-thread block
__global__ __launch_bounds__(256) void rms_combine_kernel(const float* P, float* r, int64_t M, int64_t pcols,
                                                          float D, float eps) {
  const int64_t i = int64_t(blockIdx.x) * kCombineRows + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (i < M) {
    const float* row = P + i * pcols;
    if ((pcols & 3) == 0) {  // a multiple of 4 partials per row (D a multiple of 1024): 16-byte rows
      const float4* row4 = reinterpret_cast<const float4*>(row);
      for (int64_t t = l; t < pcols / 4; t += 16) {
        const float4 v = row4[t];
        acc += (v.x + v.y) + (v.z + v.w);
      }
    } else {
      for (int64_t t = l; t < pcols; t += 16) acc += row[t];
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += shfl_xor(acc, m);
  if (l == 0 && i < M) r[i] = 1.0f / sqrtf(acc / D + eps);
}

// Block-wide sum over 256 threads, fixed order (wave shuffles, then LDS).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// Block-wide sum over 512 threads, fixed order (wave shuffles, then LDS).
__device__ __forceinline__ float block_sum512(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float t = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
  __syncthreads();
  return t;
}

// One 512-thread block per row i: s_i = sum_n dY_in y_in (fp32) and, with GR (the
// unfused baseline's row layout), gr_i = bf16(r_i g_i). The row is read in rounds of kRowUnroll x 16 bytes per
// thread of each input, all loads of a round issued before any is used (one
// round covers an N = 28672 row); dY and y are read non-temporally (about 6 % faster
// at the 8B shape).
constexpr int kRowThreads = 512;
constexpr int kRowUnroll = 7;

// 16 bytes of a stream read once (non-temporal: it need not displace cached data that
// later kernels read again, e.g. the weights and h of the data-gradient GEMM).
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
template <bool GR>
__global__ __launch_bounds__(kRowThreads) void rowstat_kernel(const uint16_t* dY, const uint16_t* y,
                                                              const uint16_t* g, const float* r, float* s,
                                                              uint16_t* gr, int64_t N, int64_t D) {
  __shared__ float red[kRowThreads / 64];
  const int64_t i = blockIdx.x;
  // bf16(r g) first: it does not wait for s, and its loads join the row's in the same round
  if constexpr (GR) {
    const float ri = r[i];
    const uint4* gs = reinterpret_cast<const uint4*>(g + i * D);
    uint4* go = reinterpret_cast<uint4*>(gr + i * D);
    for (int64_t v = threadIdx.x; v < D / 8; v += kRowThreads) {
      float f[8];
      unpack8_bf16(gs[v], f);
      const uint2 lo = pack4_bf16(ri * f[0], ri * f[1], ri * f[2], ri * f[3]);
      const uint2 hi = pack4_bf16(ri * f[4], ri * f[5], ri * f[6], ri * f[7]);
      go[v] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  const uint4* a = reinterpret_cast<const uint4*>(dY + i * N);
  const uint4* b = reinterpret_cast<const uint4*>(y + i * N);
  const int64_t n8 = N / 8;
  float acc = 0.f;
  for (int64_t base = threadIdx.x; base < n8; base += kRowThreads * kRowUnroll) {
    uint4 va[kRowUnroll], vb[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t v = base + u * kRowThreads;
      va[u] = v < n8 ? load_once(a + v) : make_uint4(0, 0, 0, 0);
      vb[u] = v < n8 ? load_once(b + v) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      float fa[8], fb[8];
      unpack8_bf16(va[u], fa);
      unpack8_bf16(vb[u], fb);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += fa[e] * fb[e];
    }
  }
  const float tot = block_sum512(acc, red);
  if (threadIdx.x == 0) s[i] = tot;
}

// Column sums out_j = sum_t P[t, j] of partials P[rows, D]: dgamma from the data-gradient GEMM's
// column partials, and s from the weight-gradient GEMM's row-dot partials (stored with the row index as
// the column). A 256-thread block covers 32 columns; its 8 row groups each sum every 8th partial row,
// four rows per round in four independent sums (four loads in flight), which are then added in a fixed
// order, as are the 8 group sums.
constexpr int kDgCols = 32, kDgGroups = 8;
__global__ __launch_bounds__(256) void colsum_kernel(const float* P, float* out, int64_t rows, int64_t D) {
  __shared__ float part[kDgGroups][kDgCols];
  const int c = threadIdx.x % kDgCols, q = threadIdx.x / kDgCols;
  const int64_t j = int64_t(blockIdx.x) * kDgCols + c;
  float acc = 0.f;
  if (j < D) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t t = q;
    for (; t + 3 * kDgGroups < rows; t += 4 * kDgGroups) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] += P[(t + u * kDgGroups) * D + j];
    }
#pragma unroll
    for (int u = 0; u < 3; ++u)  // the last rounds' rows (fewer than four)
      if (t + u * kDgGroups < rows) a[u] += P[(t + u * kDgGroups) * D + j];
    acc = (a[0] + a[1]) + (a[2] + a[3]);
  }
  part[q][c] = acc;
  __syncthreads();
  if (q == 0 && j < D) {
    float tot = 0.f;
#pragma unroll
    for (int g = 0; g < kDgGroups; ++g) tot += part[g][c];
    out[j] = tot;
  }
}

// bf16(r g) transposed for the weight-gradient GEMM, whose contraction runs over the
// rows i: grT[j, i] = bf16(r_i g_ij) for i < M and 0 for M <= i < ldt (the pad to the
// K step). A 256-thread block moves a 64 x 64 tile through LDS: 16-byte row loads of g
// and 16-byte LDS row writes, 2-byte LDS column reads, 16-byte row stores of grT (the
// transposed 2-byte writes of an earlier version met bank conflicts: about 1.3 us slower
// at the 8B shape).
__global__ __launch_bounds__(256) void gr_transpose_kernel(const uint16_t* g, const float* r, uint16_t* grT, int64_t M,
                                                           int64_t D, int64_t ldt) {
  // 64 rows i x 64 columns j through LDS, 128 bytes per row; 16-byte chunk c of row i is stored at chunk
  // c ^ s(i), s(i) = (i & 7) ^ (i >> 3): a row's 8 chunks are a permutation (16-byte row writes hit every bank
  // once per 8 lanes), and the column reads -- the same column of rows 8 q + e, q = 0 .. 7 -- fall in 8
  // different chunks.
  constexpr int kT = 64;
  __shared__ __attribute__((aligned(16))) uint16_t tile[kT * kT];
  const int64_t j0 = int64_t(blockIdx.x) * kT, i0 = int64_t(blockIdx.y) * kT;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = threadIdx.x + 256 * q, row = c >> 3, chunk = c & 7;  // row i0 + row, columns j0 + 8 chunk ..
    const int64_t i = i0 + row;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (i < M) {
      float f[8];
      unpack8_bf16(*reinterpret_cast<const uint4*>(g + i * D + j0 + 8 * chunk), f);
      const float ri = r[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= ri;
      o = make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7]));
    }
    const int s = (row & 7) ^ (row >> 3);
    *reinterpret_cast<uint4*>(&tile[row * kT + 8 * (chunk ^ s)]) = o;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = threadIdx.x + 256 * q, jr = c >> 3, ic = c & 7;  // grT row j0 + jr, columns i0 + 8 ic ..
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ra = 8 * ic + e, rb = ra + 1;
      const uint32_t a = tile[ra * kT + 8 * ((jr >> 3) ^ ((ra & 7) ^ (ra >> 3))) + (jr & 7)];
      const uint32_t b = tile[rb * kT + 8 * ((jr >> 3) ^ ((rb & 7) ^ (rb >> 3))) + (jr & 7)];
      w[e / 2] = a | (b << 16);
    }
    *reinterpret_cast<uint4*>(grT + (j0 + jr) * ldt + i0 + 8 * ic) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// SwiGLU backward: one 256-thread block per row i: s_i = sum_t Ps[i, t] (fixed order).
__global__ __launch_bounds__(256) void scombine_kernel(const float* Ps, float* s, int64_t pcols) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  float acc = 0.f;
  for (int64_t t = threadIdx.x; t < pcols; t += 256) acc += Ps[i * pcols + t];
  const float tot = block_sum256(acc, red);
  if (threadIdx.x == 0) s[i] = tot;
}

__device__ __forceinline__ float block_max256(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

// Cross-entropy combine: one 256-thread block per row. lse_i = m + log sum_t l_t
// exp(m_t - m) with m = max_t m_t over the row's (m_t, l_t) tile statistics (fixed
// order); loss_i = lse_i - target logit, 0 for an ignored row.
__global__ __launch_bounds__(256) void ce_combine_kernel(const float2* Pml, const float* tgt, const int64_t* targets,
                                                         float* lse, float* loss, int64_t pcols, int64_t V) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const float2* p = Pml + i * pcols;
  float m = -INFINITY;
  for (int64_t t = threadIdx.x; t < pcols; t += 256) m = fmaxf(m, p[t].x);
  m = block_max256(m, red);
  float l = 0.f;
  for (int64_t t = threadIdx.x; t < pcols; t += 256) {
    const float2 v = p[t];
    l += v.y * fast_exp(v.x - m);
  }
  l = block_sum256(l, red);
  if (threadIdx.x == 0) {
    const float ls = m + logf(l);
    const int64_t t = targets[i];
    lse[i] = ls;
    loss[i] = ce_valid(t, V) ? ls - tgt[i] : 0.f;
  }
}

// Rows of stored fp32 logits, one 256-thread block per row; each thread reads its
// 16-byte chunks v = tid + 256 (u + kCeUnroll q) in rounds of kCeUnroll, all loads of a
// round issued before any is used.
constexpr int kCeUnroll = 4;

// Forward: each thread keeps a running (max, sum exp) over its columns in one pass,
// then the block combines them; lse_i = m + log l, loss_i = lse_i - logit[i, t_i], 0
// for an ignored row.
__global__ __launch_bounds__(256) void ce_rows_fwd_kernel(const float* logits, const int64_t* targets, float* lse,
                                                          float* loss, int64_t V) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x, n4 = V / 4;
  const float4* lv = reinterpret_cast<const float4*>(logits + i * V);
  float m = -INFINITY, l = 0.f;
  for (int64_t v0 = threadIdx.x; v0 < n4; v0 += 256 * kCeUnroll) {
    float4 x[kCeUnroll];
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int64_t v = v0 + 256 * u;
      x[u] = v < n4 ? lv[v] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) mx = fmaxf(mx, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
    // a round always holds a real column (v0 < n4), so mx is finite
    l *= fast_exp(m - mx);
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u)
      l += (fast_exp(x[u].x - mx) + fast_exp(x[u].y - mx)) + (fast_exp(x[u].z - mx) + fast_exp(x[u].w - mx));
    m = mx;
  }
  const float mb = block_max256(m, red);
  const float lb = block_sum256(m == -INFINITY ? 0.f : l * fast_exp(m - mb), red);
  if (threadIdx.x == 0) {
    const float ls = mb + logf(lb);
    const int64_t t = targets[i];
    lse[i] = ls;
    loss[i] = ce_valid(t, V) ? ls - logits[i * V + t] : 0.f;
  }
}

// Backward: dlogits = dloss_i (exp(logit - lse_i) - [v = t_i]) stored bf16, 0 on an ignored row.
__global__ __launch_bounds__(256) void ce_rows_bwd_kernel(const float* logits, const int64_t* targets,
                                                          const float* lse, const float* dloss, uint16_t* dlogits,
                                                          int64_t V) {
  const int64_t i = blockIdx.x;
  const int64_t t = targets[i];
  const bool ok = ce_valid(t, V);
  const float ls = ok ? lse[i] : INFINITY, dl = ok ? dloss[i] : 0.f;
  const int64_t n4 = V / 4;
  const float4* lv = reinterpret_cast<const float4*>(logits + i * V);
  uint2* dv = reinterpret_cast<uint2*>(dlogits + i * V);
  for (int64_t v0 = threadIdx.x; v0 < n4; v0 += 256 * kCeUnroll) {
    float4 x[kCeUnroll];
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int64_t v = v0 + 256 * u;
      x[u] = v < n4 ? lv[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int64_t v = v0 + 256 * u;
      if (v < n4) {
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = dl * (fast_exp(xs[e] - ls) - (4 * v + e == t ? 1.0f : 0.0f));
        dv[v] = pack4_bf16(d[0], d[1], d[2], d[3]);
      }
    }
  }
}

// Split-K data gradient: G = the S slices' fp32 partial products summed in order, then the
// RMSNorm-backward algebra of the fused epilogue, da = r gamma G - (s r^2 / D) h, and the
// dgamma partials of each kSplitRows-row group, Pg[group, j] = sum of G r h. A block covers
// 1024 columns (4 per thread) of kSplitRows rows.
template <bool F32>
__global__ __launch_bounds__(256) void splitk_rmsnorm_bwd_kernel(const float* part, int S, int64_t sstride,
                                                                 const uint16_t* h, const float* r, const float* s,
                                                                 const uint16_t* gamma, void* da, float* Pg,
                                                                 int64_t M, int64_t D) {
  const int64_t j = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (j >= D) return;
  const int64_t i0 = int64_t(blockIdx.y) * kSplitRows;
  const int64_t i1 = i0 + kSplitRows < M ? i0 + kSplitRows : M;
  const float invD = 1.0f / float(D);
  float gm[4], cs[4] = {0.f, 0.f, 0.f, 0.f};
  unpack4_bf16(*reinterpret_cast<const uint2*>(gamma + j), gm);
  for (int64_t i = i0; i < i1; ++i) {
    // all S slices' loads of the row in flight before the fixed-order sum (S <= 8)
    float4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t < S) v[t] = *reinterpret_cast<const float4*>(part + t * sstride + i * D + j);
    float G[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
    for (int t = 1; t < 8; ++t)
      if (t < S) G[0] += v[t].x, G[1] += v[t].y, G[2] += v[t].z, G[3] += v[t].w;
    float hv[4], d[4];
    unpack4_bf16(*reinterpret_cast<const uint2*>(h + i * D + j), hv);
    const float ri = r[i], c2 = s[i] * ri * ri * invD;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] += G[e] * ri * hv[e];
      d[e] = ri * gm[e] * G[e] - c2 * hv[e];
    }
    if constexpr (F32) *reinterpret_cast<float4*>(static_cast<float*>(da) + i * D + j) = make_float4(d[0], d[1], d[2], d[3]);
    else *reinterpret_cast<uint2*>(static_cast<uint16_t*>(da) + i * D + j) = pack4_bf16(d[0], d[1], d[2], d[3]);
  }
  *reinterpret_cast<float4*>(Pg + int64_t(blockIdx.y) * D + j) = make_float4(cs[0], cs[1], cs[2], cs[3]);
}

// Split-K GEMM0: h = the slices' fp32 partial products summed in order + z (fp32), stored
// bf16; g = bf16(h gamma) from the fp32 h; P[i, j / 256] = the sum of squares of the fp32 h
// over each 256-column tile -- what the fused epilogue computes. A block covers 1024 columns
// (4 per thread; one wave per tile) of one row.
__global__ __launch_bounds__(256) void splitk_residual_kernel(const float* part, int S, int64_t sstride,
                                                              const uint16_t* z, const uint16_t* gamma, uint16_t* h,
                                                              uint16_t* g, float* P, int64_t D, int64_t pcols) {
  const int64_t i = blockIdx.y;
  const int64_t j = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const bool ok = j < D;  // uniform over each 16-thread group (64 columns; D is a multiple of 64)
  float ssq = 0.f;
  if (ok) {
    float hv[4], zz[4], gm[4];
    {
      const float4 v = *reinterpret_cast<const float4*>(part + i * D + j);
      hv[0] = v.x, hv[1] = v.y, hv[2] = v.z, hv[3] = v.w;
    }
    for (int t = 1; t < S; ++t) {
      const float4 v = *reinterpret_cast<const float4*>(part + t * sstride + i * D + j);
      hv[0] += v.x, hv[1] += v.y, hv[2] += v.z, hv[3] += v.w;
    }
    unpack4_bf16(*reinterpret_cast<const uint2*>(z + i * D + j), zz);
    unpack4_bf16(*reinterpret_cast<const uint2*>(gamma + j), gm);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hv[e] += zz[e];
      ssq += hv[e] * hv[e];
    }
    *reinterpret_cast<uint2*>(h + i * D + j) = pack4_bf16(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<uint2*>(g + i * D + j) = pack4_bf16(hv[0] * gm[0], hv[1] * gm[1], hv[2] * gm[2], hv[3] * gm[3]);
  }
  // a wave's 64 threads cover one 256-column tile: its partial P[i, j / 256]
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ssq += shfl_xor(ssq, m);
  if (ok && (threadIdx.x & 63) == 0) P[i * pcols + j / kBN] = ssq;
}

// Unfused SwiGLU: o = silu(gate) * up from the stored bf16 y, four pairs (16 bytes
// of y) per thread; y [M, 2F] and o [M, F] are walked as flat arrays (pair p of
// the flat o is y elements 2p, 2p + 1).
template <bool F32>
__global__ __launch_bounds__(256) void swiglu_rows_kernel(const uint16_t* y, void* o, int64_t quads) {
  for (int64_t v = int64_t(blockIdx.x) * 256 + threadIdx.x; v < quads; v += int64_t(gridDim.x) * 256) {
    float f[8];
    unpack8_bf16(reinterpret_cast<const uint4*>(y)[v], f);
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = f[2 * e] * sigmoidf_(f[2 * e]) * f[2 * e + 1];
    if constexpr (F32) {
      reinterpret_cast<float4*>(o)[v] = make_float4(q[0], q[1], q[2], q[3]);
    } else {
      reinterpret_cast<uint2*>(o)[v] = pack4_bf16(q[0], q[1], q[2], q[3]);
    }
  }
}

// Unfused SwiGLU backward: one 512-thread block per row i, from the stored bf16 dO:
// dY_2f = dO up silu'(gate), dY_2f+1 = dO silu(gate) (bf16) and s_i = sum dY y (fp32 dY,
// bf16 y).
__global__ __launch_bounds__(kRowThreads) void swiglu_bwd_rows_kernel(const uint16_t* dO, const uint16_t* y,
                                                                      uint16_t* dY, float* s, int64_t F) {
  __shared__ float red[kRowThreads / 64];
  const int64_t i = blockIdx.x;
  const uint2* ov = reinterpret_cast<const uint2*>(dO + i * F);
  const uint4* yv = reinterpret_cast<const uint4*>(y + i * 2 * F);
  uint4* dv = reinterpret_cast<uint4*>(dY + i * 2 * F);
  float part = 0.f;
  for (int64_t v = threadIdx.x; v < F / 4; v += kRowThreads) {
    float d4[4], yy[8], d[8];
    unpack4_bf16(ov[v], d4);
    unpack8_bf16(yv[v], yy);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gate = yy[2 * e], up = yy[2 * e + 1], sg = sigmoidf_(gate);
      d[2 * e] = d4[e] * up * (sg * (1.0f + gate * (1.0f - sg)));
      d[2 * e + 1] = d4[e] * (gate * sg);
      part += d[2 * e] * gate + d[2 * e + 1] * up;
    }
    const uint2 lo = pack4_bf16(d[0], d[1], d[2], d[3]), hi = pack4_bf16(d[4], d[5], d[6], d[7]);
    dv[v] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  const float tot = block_sum512(part, red);
  if (threadIdx.x == 0) s[i] = tot;
}

// Unfused: one block per row. h = t + z (fp32, stored bf16), r from the fp32 h,
// n = bf16(r h gamma) for the second GEMM.
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(const uint16_t* t, const uint16_t* z,
                                                          const uint16_t* gamma, uint16_t* h, float* r,
                                                          uint16_t* n, int64_t D, float eps) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const uint4* tv = reinterpret_cast<const uint4*>(t + i * D);
  const uint4* zv = reinterpret_cast<const uint4*>(z + i * D);
  float ssq = 0.f;
  for (int64_t v = threadIdx.x; v < D / 8; v += 256) {
    float a[8], b[8];
    unpack8_bf16(tv[v], a);
    unpack8_bf16(zv[v], b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float hv = a[e] + b[e];
      ssq += hv * hv;
    }
  }
  const float tot = block_sum256(ssq, red);
  const float ri = 1.0f / sqrtf(tot / float(D) + eps);
  if (threadIdx.x == 0) r[i] = ri;
  const uint4* gv = reinterpret_cast<const uint4*>(gamma);
  uint4* ho = reinterpret_cast<uint4*>(h + i * D);
  uint4* no = reinterpret_cast<uint4*>(n + i * D);
  for (int64_t v = threadIdx.x; v < D / 8; v += 256) {
    float a[8], b[8], gm[8], hv[8];
    unpack8_bf16(tv[v], a);
    unpack8_bf16(zv[v], b);
    unpack8_bf16(gv[v], gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = a[e] + b[e];
    uint2 lo = pack4_bf16(hv[0], hv[1], hv[2], hv[3]), hi = pack4_bf16(hv[4], hv[5], hv[6], hv[7]);
    ho[v] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    lo = pack4_bf16(ri * hv[0] * gm[0], ri * hv[1] * gm[1], ri * hv[2] * gm[2], ri * hv[3] * gm[3]);
    hi = pack4_bf16(ri * hv[4] * gm[4], ri * hv[5] * gm[5], ri * hv[6] * gm[6], ri * hv[7] * gm[7]);
    no[v] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// Unfused RMSNorm backward on a materialised bf16 G: block (bx, by) covers
// columns [2048 bx, +2048) (8 per thread) and rows [32 by, +32).
template <bool F32>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* G, const uint16_t* h, const float* r,
                                                          const float* s, const uint16_t* gamma, void* da,
                                                          float* Pg, int64_t M, int64_t D) {
  const int64_t j = int64_t(blockIdx.y) * 2048 + threadIdx.x * 8;
  if (j >= D) return;
  const int64_t i0 = int64_t(blockIdx.x) * kUnfusedBwdRows;  // row groups on x: up to 2^31 - 1 blocks
  const float invD = 1.0f / float(D);
  float gm[8], cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  unpack8_bf16(*reinterpret_cast<const uint4*>(gamma + j), gm);
  for (int64_t i = i0; i < min(M, i0 + kUnfusedBwdRows); ++i) {
    float gv[8], hv[8], d[8];
    unpack8_bf16(*reinterpret_cast<const uint4*>(G + i * D + j), gv);
    unpack8_bf16(*reinterpret_cast<const uint4*>(h + i * D + j), hv);
    const float ri = r[i], c2 = s[i] * ri * ri * invD;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      d[e] = ri * gm[e] * gv[e] - c2 * hv[e];
      cs[e] += gv[e] * ri * hv[e];
    }
    if constexpr (F32) {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(da) + i * D + j);
      o[0] = make_float4(d[0], d[1], d[2], d[3]);
      o[1] = make_float4(d[4], d[5], d[6], d[7]);
    } else {
      const uint2 lo = pack4_bf16(d[0], d[1], d[2], d[3]), hi = pack4_bf16(d[4], d[5], d[6], d[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(da) + i * D + j) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  float4* o = reinterpret_cast<float4*>(Pg + int64_t(blockIdx.x) * D + j);
  o[0] = make_float4(cs[0], cs[1], cs[2], cs[3]);
  o[1] = make_float4(cs[4], cs[5], cs[6], cs[7]);
}

// ----------------------------------------------------------- launchers

template <bool A_K, bool B_K, class Epi>
hipError_t launch_gemm(const GemmShape& p, const Epi& epi, hipStream_t st) {
  const int64_t blocks = ceil_div(p.M, kBM) * ceil_div(p.N, kBN);
  const int64_t slices = p.kslice > 0 ? ceil_div(p.K, p.kslice) : 1;
  hipLaunchKernelGGL((gemm_kernel<A_K, B_K, Epi>), dim3(unsigned(blocks), unsigned(slices)), dim3(kThreads), 0, st, p,
                     epi);
  return hipGetLastError();
}

template <bool A_K, bool B_K>
hipError_t launch_store(const GemmShape& p, void* C, int64_t ldc, bool f32, hipStream_t st) {
  if (f32) return launch_gemm<A_K, B_K>(p, EpiStore<true>{C, ldc, p.M}, st);
  return launch_gemm<A_K, B_K>(p, EpiStore<false>{C, ldc, p.M}, st);
}

hipError_t gemm_plain(const GemmShape& p, bool a_k, bool b_k, void* C, int64_t ldc, bool f32, hipStream_t st) {
  if (a_k && b_k) return launch_store<true, true>(p, C, ldc, f32, st);
  if (a_k && !b_k) return launch_store<true, false>(p, C, ldc, f32, st);
  if (!a_k && b_k) return launch_store<false, true>(p, C, ldc, f32, st);
  return launch_store<false, false>(p, C, ldc, f32, st);
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// bf16(r g) transposed into grT [D, gr_cols(M)] for the weight-gradient GEMM dW1 = bf16(r g)^T @ dY.
hipError_t gr_transpose(const uint16_t* g, const float* r, uint16_t* grT, int64_t M, int64_t D, hipStream_t st) {
  const int64_t ldt = gr_cols(M);  // ldt / 64 <= 2^22 / 64 = 65536 blocks, the device's grid-y limit
  hipLaunchKernelGGL(gr_transpose_kernel, dim3(unsigned(D / 64), unsigned(ldt / 64)), dim3(256), 0, st, g, r, grT, M, D,
                     ldt);
  return hipGetLastError();
}

// Unfused baseline: s and bf16(r g) in row layout from one row kernel.
hipError_t bwd_rowstat_rows(const coda_bwd_args_t* a, uint16_t* gr, hipStream_t st) {
  hipLaunchKernelGGL(rowstat_kernel<true>, dim3(unsigned(a->M)), dim3(kRowThreads), 0, st, (const uint16_t*)a->dY,
                     (const uint16_t*)a->y, (const uint16_t*)a->g, a->r, a->s, gr, a->N, a->D);
  return hipGetLastError();
}

hipError_t bwd_wgrad(const coda_bwd_args_t* a, const uint16_t* gr, hipStream_t st) {
  // C = dW1 [D, N]: rows j (m index) from gr^T (m contiguous), columns n from dY (n contiguous), K = M
  const GemmShape p{a->D, a->N, a->M, gr, a->D, a->dY, a->N};
  return gemm_plain(p, false, false, a->dW1, a->N, a->dW1_dtype == CODA_F32, st);
}

// The fused path's weight gradient on the transposed bf16(r g): A(m=j, k=i) = grT[j, i] (k contiguous;
// zero past M up to the K step), B(k=i, n) = dY[i, n] (n contiguous; rows past M read as 0), K = M.
// Its prologue finishes dgamma from the partials Pg[rows, D].
hipError_t bwd_wgrad_dgamma(const coda_bwd_args_t* a, const uint16_t* grT, const float* Pg, int64_t rows,
                            hipStream_t st) {
  const GemmShape p{a->D, a->N, a->M, grT, gr_cols(a->M), a->dY, a->N};
  if (a->dW1_dtype == CODA_F32)
    return launch_gemm<true, false>(p, EpiStoreDgamma<true>{a->dW1, a->N, p.M, Pg, a->dgamma, rows, a->D}, st);
  return launch_gemm<true, false>(p, EpiStoreDgamma<false>{a->dW1, a->N, p.M, Pg, a->dgamma, rows, a->D}, st);
}

hipError_t colsum(const float* P, float* out, int64_t rows, int64_t D, hipStream_t st) {
  hipLaunchKernelGGL(colsum_kernel, dim3(unsigned(ceil_div(D, kDgCols))), dim3(256), 0, st, P, out, rows, D);
  return hipGetLastError();
}
hipError_t bwd_dgamma(const float* Pg, int64_t rows, const coda_bwd_args_t* a, hipStream_t st) {
  return colsum(Pg, a->dgamma, rows, a->D, st);
}

// The fused chain backward's weight gradient (dW1 only; its dgamma is combined after the data gradient),
// with s's partials Ps as side work where bwd_rowdot(D) holds. Shapes as in bwd_wgrad_dgamma.
hipError_t bwd_wgrad_rowdot(const coda_bwd_args_t* a, const uint16_t* grT, float* Ps, hipStream_t st) {
  const GemmShape p{a->D, a->N, a->M, grT, gr_cols(a->M), a->dY, a->N};
  const bool f32 = a->dW1_dtype == CODA_F32;
  if (!bwd_rowdot(a->D)) return launch_store<true, false>(p, a->dW1, a->N, f32, st);
  const int ndt = int(ceil_div(a->D, kBN));
  if (f32)
    return launch_gemm<true, false>(p, EpiStoreRowDot<true>{a->dW1, a->N, p.M, (const uint16_t*)a->y, Ps, a->N, a->M, ndt}, st);
  return launch_gemm<true, false>(p, EpiStoreRowDot<false>{a->dW1, a->N, p.M, (const uint16_t*)a->y, Ps, a->N, a->M, ndt}, st);
}

// s from the side work's partials, or (fewer than 16 row tiles) from a row kernel over dY and y.
hipError_t bwd_s(const coda_bwd_args_t* a, const float* Ps, hipStream_t st) {
  if (bwd_rowdot(a->D)) return colsum(Ps, a->s, rowdot_cols(a->N), a->M, st);
  hipLaunchKernelGGL(rowstat_kernel<false>, dim3(unsigned(a->M)), dim3(kRowThreads), 0, st, (const uint16_t*)a->dY,
                     (const uint16_t*)a->y, (const uint16_t*)a->g, a->r, a->s, (uint16_t*)nullptr, a->N, a->D);
  return hipGetLastError();
}

// Raster of the data-gradient GEMM (both operands k-contiguous, contraction over N): an
// XCD's 32 concurrent tiles as 8 tile-rows x 4 tile-columns ran it about 1.5 % faster than
// the 4 x 8 of the other GEMMs, which in turn suits those better.
constexpr int kDgradGroupM = 8;

// The data gradient with its RMSNorm-backward epilogue; with few rows (dgrad_split) the
// contraction is split over S block rows into fp32 partials `part` and a row kernel finishes.
hipError_t bwd_dgrad(const coda_bwd_args_t* a, float* Pg, float* part, hipStream_t st) {
  // G = dY @ W1^T: A = dY [M, N] (k contiguous), B(k=n, j) = W1[j, n] (k contiguous)
  const KSplit ks = dgrad_split(a->M, a->D, a->N);
  if (ks.S > 1) {
    const int64_t sstride = a->M * a->D;
    const GemmShape pp{a->M, a->D, a->N, a->dY, a->N, a->W1, a->N, ks.kslice};
    hipError_t e = launch_gemm<true, true>(pp, EpiPartialF32{part, a->D, a->M, sstride}, st);
    if (e != hipSuccess) return e;
    const dim3 grid(unsigned(ceil_div(a->D, 1024)), unsigned(ceil_div(a->M, kSplitRows)));
    if (a->da_dtype == CODA_F32)
      hipLaunchKernelGGL(splitk_rmsnorm_bwd_kernel<true>, grid, dim3(256), 0, st, (const float*)part, int(ks.S), sstride,
                         (const uint16_t*)a->h, a->r, a->s, (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D);
    else
      hipLaunchKernelGGL(splitk_rmsnorm_bwd_kernel<false>, grid, dim3(256), 0, st, (const float*)part, int(ks.S), sstride,
                         (const uint16_t*)a->h, a->r, a->s, (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D);
    return hipGetLastError();
  }
  const GemmShape pd{a->M, a->D, a->N, a->dY, a->N, a->W1, a->N, 0, kDgradGroupM};
  if (a->da_dtype == CODA_F32)
    return launch_gemm<true, true>(pd, EpiRmsNormBwd<true>{(const uint16_t*)a->h, a->r, a->s, (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D}, st);
  return launch_gemm<true, true>(pd, EpiRmsNormBwd<false>{(const uint16_t*)a->h, a->r, a->s, (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D}, st);
}

coda_status_t to_status(hipError_t e) { return e == hipSuccess ? CODA_OK : CODA_ERR_HIP; }

// The fused backward's workspace regions (layout in coda_internal.h).
struct BwdWorkspace {
  uint16_t* gr;     // bf16(r g) [M, D]
  float* Pg;        // dgamma partials [pg_rows, D]
  float* part;      // split-K partial products [S, M, D] (split only)
  int64_t pg_rows;
};
BwdWorkspace bwd_workspace(void* ws, int64_t M, int64_t D, int64_t N) {
  return {reinterpret_cast<uint16_t*>(ws), reinterpret_cast<float*>(ws_at(ws, bwd_ws_gr(M, D))),
          reinterpret_cast<float*>(ws_at(ws, bwd_ws_part(M, D, N))), bwd_pg_rows(M, D, N)};
}

// dh and dW from the bf16 dlogits (shared by the fused and the unfused backward).
hipError_t ce_bwd_products(const coda_ce_bwd_args_t* a, hipStream_t st) {
  // dh [M, D] = dlogits @ W: A = dlogits [M, V] (k contiguous), B(k=v, d) = W[v, d] (n contiguous)
  const GemmShape pd{a->M, a->D, a->V, a->dlogits, a->V, a->W, a->D};
  hipError_t e = gemm_plain(pd, true, false, a->dh, a->D, a->dh_dtype == CODA_F32, st);
  if (e != hipSuccess) return e;
  // dW [V, D] = dlogits^T @ h: A(m=v, k=i) = dlogits[i, v] (m contiguous), B(k=i, d) = h[i, d] (n contiguous), K = M
  const GemmShape pw{a->V, a->D, a->M, a->dlogits, a->V, a->h, a->D};
  return gemm_plain(pw, false, false, a->dW, a->D, a->dW_dtype == CODA_F32, st);
}

// GEMM1 g @ W1 with a row-scale epilogue Epi<F32, FOLD> (EpiRowScale or EpiRowScaleSwiglu), whose row scales
// are combined from the partials P in the epilogue where fwd_folds_combine says so, else read from r;
// `more` are the epilogue's fields after its row scales.
template <template <bool, bool> class Epi, class... More>
hipError_t launch_gemm1(const coda_fwd_args_t* a, const float* P, bool f32, hipStream_t st, More... more) {
  const GemmShape p1{a->M, a->N, a->D, a->g, a->D, a->W1, a->N};
  const int64_t pcols = ssq_cols(a->D);
  if (fwd_folds_combine(a->M, a->D, a->N)) {
    const RowScaleSrc<true> rs{a->r, P, a->M, pcols, float(a->D), a->eps};
    return f32 ? launch_gemm<true, false>(p1, Epi<true, true>{rs, more...}, st)
               : launch_gemm<true, false>(p1, Epi<false, true>{rs, more...}, st);
  }
  const RowScaleSrc<false> rs{a->r, nullptr, a->M, pcols, float(a->D), a->eps};
  return f32 ? launch_gemm<true, false>(p1, Epi<true, false>{rs, more...}, st)
             : launch_gemm<true, false>(p1, Epi<false, false>{rs, more...}, st);
}

// Stage `stage` of the fused forward (0 GEMM0 + epilogue, 1 r combine, 2 GEMM1 + row scale) with the
// sum-of-squares partials P [M, ceil(D / 256)]; part: room for GEMM0's split-K partial products when its tiles
// cannot fill the chip, or nullptr to never split (the no-allocation entry point).
hipError_t fwd_stage(int stage, const coda_fwd_args_t* a, float* P, float* part, hipStream_t st) {
  const int64_t pcols = ssq_cols(a->D);
  if (stage == 0) {  // GEMM0 x @ W0 with the residual / h / g / sum-of-squares epilogue
    const KSplit ks = part != nullptr ? gemm0_split(a->M, a->K0, a->D) : KSplit{1, 0};
    if (ks.S > 1) {  // few rows: split the contraction, then a row kernel does the epilogue's work
      const int64_t sstride = a->M * a->D;
      const GemmShape pp{a->M, a->D, a->K0, a->x, a->K0, a->W0, a->D, ks.kslice};
      hipError_t e = launch_gemm<true, false>(pp, EpiPartialF32{part, a->D, a->M, sstride}, st);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(splitk_residual_kernel, dim3(unsigned(ceil_div(a->D, 1024)), unsigned(a->M)), dim3(256), 0, st,
                         (const float*)part, int(ks.S), sstride, (const uint16_t*)a->z, (const uint16_t*)a->gamma,
                         (uint16_t*)a->h, (uint16_t*)a->g, P, a->D, pcols);
      return hipGetLastError();
    }
    const GemmShape p0{a->M, a->D, a->K0, a->x, a->K0, a->W0, a->D};
    return launch_gemm<true, false>(
        p0, EpiResidualSsq{(const uint16_t*)a->z, (const uint16_t*)a->gamma, (uint16_t*)a->h, (uint16_t*)a->g, P, a->M, a->D, pcols}, st);
  }
  if (stage == 1) {  // partial sums of squares -> r, unless GEMM1's epilogue combines them itself
    if (fwd_folds_combine(a->M, a->D, a->N)) return hipSuccess;
    hipLaunchKernelGGL(rms_combine_kernel, dim3(unsigned(ceil_div(a->M, kCombineRows))), dim3(256), 0, st, P, a->r, a->M,
                       pcols, float(a->D), a->eps);
    return hipGetLastError();
  }
  // GEMM1 g @ W1 with the row-scale epilogue
  return launch_gemm1<EpiRowScale>(a, P, a->y_dtype == CODA_F32, st, a->y, a->N);
}

// ------------------------------------------------- no-allocation forward
// coda_fwd_noalloc keeps its partials P in this file-scope device array (one copy per GPU, held until
// the process ends) instead of a caller's workspace. In host code `scratch` names a host-side stand-in,
// not the device memory: every use goes through the address hipGetSymbolAddress returns for the
// device that runs the call, looked up once per device and kept.
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the device that `st` belongs to.
hipError_t scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;   // the lookup is per current device
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace coda

using namespace coda;

extern "C" {

coda_status_t coda_fwd_stage(int stage, const coda_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_fwd(a, ws, ws_bytes);
  if (v != CODA_OK) return v;
  if (stage < 0 || stage >= CODA_FWD_STAGES) return CODA_ERR_ARG;
  float* part = reinterpret_cast<float*>(ws_at(ws, fwd_ws_p(a->M, a->D)));
  return to_status(fwd_stage(stage, a, reinterpret_cast<float*>(ws), part, static_cast<hipStream_t>(stream)));
}

coda_status_t coda_fwd(const coda_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  for (int s = 0; s < CODA_FWD_STAGES; ++s) {
    const coda_status_t v = coda_fwd_stage(s, a, ws, ws_bytes, stream);
    if (v != CODA_OK) return v;
  }
  return CODA_OK;
}

coda_status_t coda_fwd_noalloc(const coda_fwd_args_t* a, void* stream) {
  coda_status_t v = coda_validate_fwd_noalloc(a);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* P = nullptr;
  if (scratch_address(st, &P) != hipSuccess) return CODA_ERR_HIP;
  // P is written in full (every row's ceil(D / 256) partials) by stage 0 before any later stage reads it, so the
  // previous call's contents need no clearing
  for (int s = 0; s < CODA_FWD_STAGES; ++s)
    if (fwd_stage(s, a, static_cast<float*>(P), nullptr, st) != hipSuccess) return CODA_ERR_HIP;
  return CODA_OK;
}

coda_status_t coda_bwd_stage(int stage, const coda_bwd_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_bwd(a, ws, ws_bytes);
  if (v != CODA_OK) return v;
  if (stage < 0 || stage >= CODA_BWD_STAGES) return CODA_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BwdWorkspace w = bwd_workspace(ws, a->M, a->D, a->N);
  float* Ps = reinterpret_cast<float*>(ws_at(ws, bwd_ws(a->M, a->D, a->N)));
  switch (stage) {
    case 0: return to_status(gr_transpose((const uint16_t*)a->g, a->r, w.gr, a->M, a->D, st));
    case 1: return to_status(bwd_wgrad_rowdot(a, w.gr, Ps, st));
    case 2: return to_status(bwd_s(a, Ps, st));
    case 3: return to_status(bwd_dgrad(a, w.Pg, w.part, st));
    default: return to_status(bwd_dgamma(w.Pg, w.pg_rows, a, st));
  }
}

coda_status_t coda_bwd(const coda_bwd_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  for (int s = 0; s < CODA_BWD_STAGES; ++s) {
    const coda_status_t v = coda_bwd_stage(s, a, ws, ws_bytes, stream);
    if (v != CODA_OK) return v;
  }
  return CODA_OK;
}

coda_status_t coda_unfused_ref(coda_op_t op, const void* args, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_unfused(op, args, ws, ws_bytes);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (op == CODA_OP_FWD) {
    const coda_fwd_args_t* a = static_cast<const coda_fwd_args_t*>(args);
    const size_t md = align256(size_t(a->M) * size_t(a->D) * 2);
    uint16_t* t = reinterpret_cast<uint16_t*>(ws);
    uint16_t* n = reinterpret_cast<uint16_t*>(ws_at(ws, md));
    const GemmShape p0{a->M, a->D, a->K0, a->x, a->K0, a->W0, a->D};
    hipError_t e = gemm_plain(p0, true, false, t, a->D, false, st);
    if (e != hipSuccess) return CODA_ERR_HIP;
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(unsigned(a->M)), dim3(256), 0, st, t, (const uint16_t*)a->z,
                       (const uint16_t*)a->gamma, (uint16_t*)a->h, a->r, n, a->D, a->eps);
    if ((e = hipGetLastError()) != hipSuccess) return CODA_ERR_HIP;
    const GemmShape p1{a->M, a->N, a->D, n, a->D, a->W1, a->N};
    return to_status(gemm_plain(p1, true, false, a->y, a->N, a->y_dtype == CODA_F32, st));
  }
  if (op == CODA_OP_FWD_SWIGLU) {
    const coda_fwd_swiglu_args_t* a = static_cast<const coda_fwd_swiglu_args_t*>(args);
    if ((v = coda_fwd(&a->chain, ws, ws_bytes, stream)) != CODA_OK) return v;
    const int64_t quads = a->chain.M * (a->chain.N / 2) / 4;
    const unsigned grid = unsigned(std::min<int64_t>(ceil_div(quads, 256), 16384));
    if (a->o_dtype == CODA_F32)
      hipLaunchKernelGGL(swiglu_rows_kernel<true>, dim3(grid), dim3(256), 0, st, (const uint16_t*)a->chain.y, a->o, quads);
    else
      hipLaunchKernelGGL(swiglu_rows_kernel<false>, dim3(grid), dim3(256), 0, st, (const uint16_t*)a->chain.y, a->o, quads);
    return to_status(hipGetLastError());
  }
  if (op == CODA_OP_BWD_SWIGLU) {
    const coda_bwd_swiglu_args_t* a = static_cast<const coda_bwd_swiglu_args_t*>(args);
    const int64_t F = a->N / 2;
    const BwdWorkspace w = bwd_workspace(ws, a->M, a->D, a->N);
    uint16_t* gr = w.gr;
    uint16_t* dO = reinterpret_cast<uint16_t*>(ws_at(ws, bwd_ws(a->M, a->D, a->N)));
    const GemmShape po{a->M, F, a->E, a->dOut, a->E, a->W2, a->E};
    hipError_t e = gemm_plain(po, true, true, dO, F, false, st);
    if (e != hipSuccess) return CODA_ERR_HIP;
    hipLaunchKernelGGL(swiglu_bwd_rows_kernel, dim3(unsigned(a->M)), dim3(kRowThreads), 0, st, (const uint16_t*)dO,
                       (const uint16_t*)a->y, (uint16_t*)a->dY, a->s, F);
    if ((e = hipGetLastError()) != hipSuccess) return CODA_ERR_HIP;
    if ((e = gr_transpose((const uint16_t*)a->g, a->r, gr, a->M, a->D, st)) != hipSuccess) return CODA_ERR_HIP;
    const coda_bwd_args_t c{a->M, a->D, a->N, a->dY, a->y, a->h, a->g, a->r, a->gamma, a->W1,
                            a->da, a->dgamma, a->dW1, a->s, a->da_dtype, a->dW1_dtype};
    if ((e = bwd_dgrad(&c, w.Pg, w.part, st)) != hipSuccess) return CODA_ERR_HIP;
    if ((e = bwd_wgrad_dgamma(&c, gr, w.Pg, w.pg_rows, st)) != hipSuccess) return CODA_ERR_HIP;
    const GemmShape pw{F, a->E, a->M, a->o, F, a->dOut, a->E};
    return to_status(gemm_plain(pw, false, false, a->dW2, a->E, a->dW2_dtype == CODA_F32, st));
  }
  if (op == CODA_OP_CE_FWD || op == CODA_OP_CE_BWD) {
    // the fp32 logits h @ W^T stored in the workspace, then a row kernel
    const coda_ce_fwd_args_t* f = static_cast<const coda_ce_fwd_args_t*>(args);
    const coda_ce_bwd_args_t* b = static_cast<const coda_ce_bwd_args_t*>(args);
    const int64_t M = op == CODA_OP_CE_FWD ? f->M : b->M, D = op == CODA_OP_CE_FWD ? f->D : b->D;
    const int64_t V = op == CODA_OP_CE_FWD ? f->V : b->V;
    const void* h = op == CODA_OP_CE_FWD ? f->h : b->h;
    const void* W = op == CODA_OP_CE_FWD ? f->W : b->W;
    float* logits = reinterpret_cast<float*>(ws);
    const GemmShape p{M, V, D, h, D, W, D};
    hipError_t e = gemm_plain(p, true, true, logits, V, true, st);
    if (e != hipSuccess) return CODA_ERR_HIP;
    if (op == CODA_OP_CE_FWD) {
      hipLaunchKernelGGL(ce_rows_fwd_kernel, dim3(unsigned(M)), dim3(256), 0, st, (const float*)logits, f->targets,
                         f->lse, f->loss, V);
      return to_status(hipGetLastError());
    }
    hipLaunchKernelGGL(ce_rows_bwd_kernel, dim3(unsigned(M)), dim3(256), 0, st, (const float*)logits, b->targets,
                       b->lse, b->dloss, (uint16_t*)b->dlogits, V);
    if ((e = hipGetLastError()) != hipSuccess) return CODA_ERR_HIP;
    return to_status(ce_bwd_products(b, st));
  }
  const coda_bwd_args_t* a = static_cast<const coda_bwd_args_t*>(args);
  const size_t md = align256(size_t(a->M) * size_t(a->D) * 2);
  uint16_t* gr = reinterpret_cast<uint16_t*>(ws);
  uint16_t* G = reinterpret_cast<uint16_t*>(ws_at(ws, md));
  float* Pg = reinterpret_cast<float*>(ws_at(ws, 2 * md));
  hipError_t e = bwd_rowstat_rows(a, gr, st);
  if (e != hipSuccess) return CODA_ERR_HIP;
  const GemmShape pd{a->M, a->D, a->N, a->dY, a->N, a->W1, a->N, 0, kDgradGroupM};
  if ((e = gemm_plain(pd, true, true, G, a->D, false, st)) != hipSuccess) return CODA_ERR_HIP;
  const dim3 grid(unsigned(ceil_div(a->M, kUnfusedBwdRows)), unsigned(ceil_div(a->D, 2048)));
  if (a->da_dtype == CODA_F32)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<true>, grid, dim3(256), 0, st, G, (const uint16_t*)a->h, a->r, a->s,
                       (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<false>, grid, dim3(256), 0, st, G, (const uint16_t*)a->h, a->r, a->s,
                       (const uint16_t*)a->gamma, a->da, Pg, a->M, a->D);
  if ((e = hipGetLastError()) != hipSuccess) return CODA_ERR_HIP;
  if ((e = bwd_dgamma(Pg, ceil_div(a->M, kUnfusedBwdRows), a, st)) != hipSuccess) return CODA_ERR_HIP;
  return to_status(bwd_wgrad(a, gr, st));
}

coda_status_t coda_fwd_swiglu(const coda_fwd_swiglu_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_fwd_swiglu(a, ws, ws_bytes);
  if (v != CODA_OK) return v;
  const coda_fwd_args_t* c = &a->chain;
  for (int s = 0; s < 2; ++s)  // GEMM0 with its epilogue, then r
    if ((v = coda_fwd_stage(s, c, ws, ws_bytes, stream)) != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // P leads the workspace
  return to_status(launch_gemm1<EpiRowScaleSwiglu>(c, static_cast<const float*>(ws), a->o_dtype == CODA_F32, st,
                                                   c->y, a->o, c->N));
}

coda_status_t coda_bwd_swiglu(const coda_bwd_swiglu_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_bwd_swiglu(a, ws, ws_bytes);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t F = a->N / 2, pcols = swiglu_s_cols(a->N);
  const BwdWorkspace w = bwd_workspace(ws, a->M, a->D, a->N);
  uint16_t* gr = w.gr;
  float* Ps = reinterpret_cast<float*>(ws_at(ws, bwd_ws(a->M, a->D, a->N)));
  // dO = dOut @ W2^T with the SwiGLU-backward epilogue: A = dOut [M, E], B(k=e, f) = W2[f, e] (both k contiguous)
  const GemmShape po{a->M, F, a->E, a->dOut, a->E, a->W2, a->E};
  hipError_t e = launch_gemm<true, true>(po, EpiSwigluBwd{(const uint16_t*)a->y, (uint16_t*)a->dY, Ps, a->M, F, pcols}, st);
  if (e != hipSuccess) return CODA_ERR_HIP;
  hipLaunchKernelGGL(scombine_kernel, dim3(unsigned(a->M)), dim3(256), 0, st, Ps, a->s, pcols);
  if ((e = hipGetLastError()) != hipSuccess) return CODA_ERR_HIP;
  if ((e = gr_transpose((const uint16_t*)a->g, a->r, gr, a->M, a->D, st)) != hipSuccess) return CODA_ERR_HIP;
  // the chain's backward on dY, with s and bf16(r g) already in place
  const coda_bwd_args_t c{a->M, a->D, a->N, a->dY, a->y, a->h, a->g, a->r, a->gamma, a->W1,
                          a->da, a->dgamma, a->dW1, a->s, a->da_dtype, a->dW1_dtype};
  if ((e = bwd_dgrad(&c, w.Pg, w.part, st)) != hipSuccess) return CODA_ERR_HIP;
  if ((e = bwd_wgrad_dgamma(&c, gr, w.Pg, w.pg_rows, st)) != hipSuccess) return CODA_ERR_HIP;
  // dW2 [F, E] = o^T @ dOut: A(m=f, k=i) = o[i, f] (m contiguous), B(k=i, n=e) = dOut[i, e] (n contiguous), K = M
  const GemmShape pw{F, a->E, a->M, a->o, F, a->dOut, a->E};
  return to_status(gemm_plain(pw, false, false, a->dW2, a->E, a->dW2_dtype == CODA_F32, st));
}

coda_status_t coda_ce_fwd(const coda_ce_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  coda_status_t v = coda_validate_ce_fwd(a, ws, ws_bytes);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t pcols = ce_stat_cols(a->V);
  float2* Pml = reinterpret_cast<float2*>(ws);
  float* tgt = reinterpret_cast<float*>(ws_at(ws, align256(size_t(a->M) * size_t(pcols) * 8)));
  // logits = h @ W^T: A = h [M, D], B(k=d, v) = W[v, d] (both k contiguous)
  const GemmShape p{a->M, a->V, a->D, a->h, a->D, a->W, a->D};
  hipError_t e = a->logits != nullptr
                     ? launch_gemm<true, true>(p, EpiCeStats<true>{a->targets, Pml, tgt, a->logits, a->M, a->V, pcols}, st)
                     : launch_gemm<true, true>(p, EpiCeStats<false>{a->targets, Pml, tgt, nullptr, a->M, a->V, pcols}, st);
  if (e != hipSuccess) return CODA_ERR_HIP;
  hipLaunchKernelGGL(ce_combine_kernel, dim3(unsigned(a->M)), dim3(256), 0, st, (const float2*)Pml, (const float*)tgt,
                     a->targets, a->lse, a->loss, pcols, a->V);
  return to_status(hipGetLastError());
}

coda_status_t coda_ce_bwd(const coda_ce_bwd_args_t* a, void* stream) {
  coda_status_t v = coda_validate_ce_bwd(a);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a->logits != nullptr) {  // the forward's stored logits: a row kernel instead of the GEMM
    hipLaunchKernelGGL(ce_rows_bwd_kernel, dim3(unsigned(a->M)), dim3(256), 0, st, a->logits, a->targets, a->lse,
                       a->dloss, static_cast<uint16_t*>(a->dlogits), a->V);
    e = hipGetLastError();
  } else {  // recomputed logits with the dlogits epilogue
    const GemmShape p{a->M, a->V, a->D, a->h, a->D, a->W, a->D};
    e = launch_gemm<true, true>(
        p, EpiCeBwd{a->targets, a->lse, a->dloss, static_cast<uint16_t*>(a->dlogits), a->M, a->V}, st);
  }
  if (e != hipSuccess) return CODA_ERR_HIP;
  return to_status(ce_bwd_products(a, st));
}

coda_status_t coda_bwd_gemm0(const coda_bwd_gemm0_args_t* a, void* stream) {
  coda_status_t v = coda_validate_bwd_gemm0(a);
  if (v != CODA_OK) return v;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // dx [M,K0] = dh @ W0^T: A = dh [M,D] (k contiguous), B(k=j, n=k0) = W0[k0, j] (k contiguous)
  const GemmShape px{a->M, a->K0, a->D, a->dh, a->D, a->W0, a->D};
  hipError_t e = gemm_plain(px, true, true, a->dx, a->K0, a->dx_dtype == CODA_F32, st);
  if (e != hipSuccess) return CODA_ERR_HIP;
  // dW0 [K0,D] = x^T @ dh: A(m=k0, k=i) = x[i, k0] (m contiguous), B(k=i, n=j) = dh[i, j] (n contiguous), K = M
  const GemmShape pw{a->K0, a->D, a->M, a->x, a->K0, a->dh, a->D};
  return to_status(gemm_plain(pw, false, false, a->dW0, a->D, a->dW0_dtype == CODA_F32, st));
}

coda_status_t coda_gemm(const coda_gemm_args_t* a, void* stream) {
  coda_status_t v = coda_validate_gemm(a);
  if (v != CODA_OK) return v;
  const GemmShape p{a->M, a->N, a->K, a->A, a->lda, a->B, a->ldb};
  return to_status(gemm_plain(p, a->a_layout == CODA_ROW, a->b_layout == CODA_COL, a->C, a->ldc,
                              a->c_dtype == CODA_F32, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
