// Shared pieces of the two attention-backward kernels (fa_backward.hip:
// dK, dV; fa_backward_dq.hip: dQ): tile geometry, the LDS swizzle, DMA and
// LDS-read helpers, the order of products inside a pipeline step, the work
// order and the mask helpers.  Everything sits in an anonymous namespace, so
// each translation unit has its own copy.
#pragma once

#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

// dQ of the backward pass (fa_backward_dq.hip), d = 64 or 128; it also writes
// the per-row workspace terms that the dK, dV kernel reads, so it runs first.
hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t stream);

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;

constexpr int kBThreads = 256;                 // 4 waves, one per SIMD
constexpr int kBWaves = 4;
constexpr int kWaveRows = 32;                  // keys (dkdv) or query rows (dq) of one wave
constexpr int kUnit = kBWaves * kWaveRows;     // keys or rows of one workgroup
constexpr int kTile = 64;                      // rows of a streamed tile
constexpr int kRing = 4;                       // tile slots in LDS
constexpr int kLook = 4;                       // operand fragments read ahead of their product
constexpr int kRsrcWord3 = 0x00020000;         // raw buffer, 32-bit data format
constexpr int kFar = 1 << 28;                  // an unbounded side of a mask interval

template <int D, int NW = kBWaves>
struct BTile {
  static constexpr int kCh = D / 8;                       // 16-byte chunks per row
  static constexpr int kRowB = D * 2;                     // bytes per row in LDS
  static constexpr int kBytes = kTile * kRowB;            // one tensor's tile
  static constexpr int kLoads = kBytes / 1024 / NW;  // 1 KB DMA loads per wave per tensor
  static constexpr int kVec = kTile * 4;                  // one fp32 value per tile row
  static_assert(kBytes % (1024 * NW) == 0, "tile must split evenly over the waves");
};

// The 32 rows behind a 32x32 score accumulator enter in this order, so that
// lane half h, register r holds logical row 16 (r / 8) + 8 h + (r % 8).
__device__ __forceinline__ int pi_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Tiles are read two ways: by rows (16 lanes take one 16-byte chunk of 16
// consecutive rows) and transposed (32 lanes take 4 chunks of 4 consecutive
// rows).  Chunk c of row r sits at c ^ bswz(r): within any 16 aligned rows the
// swizzles are distinct (row reads hit 16 different bank groups), and within
// any 4 aligned rows the group of 4 chunks they select differs (transposed
// reads too).  At d = 64 two rows share a 256-byte bank line, so the row
// parity already separates neighbours and the swizzle uses r >> 1.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

__device__ __forceinline__ u32x4_t rsrc_of(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcWord3;
  return r;
}

// 16 (or 4) bytes per lane from the buffer at byte offset voff straight into
// LDS at lds_base + 16 (or 4) * lane; offsets past the descriptor's size read
// zeros.  Inline assembly keeps the loads out of the compiler's wait
// tracking: the only waits for them are the explicit vmcnt waits before the
// barriers, so LDS reads of other ring slots never wait for them.
__device__ __forceinline__ void dma_b128(const u32x4_t& rs, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void dma_b32(const u32x4_t& rs, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(lds_base)
      : "memory");
}

// Four 16-byte-per-lane loads into four consecutive 1 KB LDS blocks under one
// M0 setting: the instruction offset (k * 1024) moves the LDS destination and
// the memory address together, so voff[k] carries the memory offset minus it.
__device__ __forceinline__ void dma_b128x4(const u32x4_t& rs, uint32_t v0, uint32_t v1, uint32_t v2,
                                           uint32_t v3, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rs), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)p);
}

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier with no implicit wait (see the DMA helpers).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8_t lds_row(const char* p) {
  return *(const lds_bf16x8_t*)((const lds_void_t*)p);
}
__device__ __forceinline__ bf16x8_t lds_tr(const char* lo, const char* hi) {
  const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_void_t*)lo));
  const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_void_t*)hi));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ f32x4_t lds_f4(const char* p) {
  return *(const lds_f32x4_t*)((const lds_void_t*)p);
}

// Anchor a value at this point of the program: the optimizer may not sink its
// computation past here (sched_barrier alone binds only the final scheduler)
__device__ __forceinline__ void anchor(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void anchor(uint32_t x) { asm volatile("" ::"v"(x)); }

// two floats to a bf16 pair (round to nearest even) in one conversion
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2v_t));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane byte offsets of the two operand reads inside one tile.
//  row[kk]: the row-wise fragment of 32-row block 0 (rows in pi order) with
//           d = 16 kk + 8 h .. + 7 (the reduction index of S and dP);
//  tlo/thi[db]: the transposed fragment of 16-row slice 0, columns
//           32 db + l % 32, rows 8 h .. + 3 and 8 h + 4 .. + 7.
// Other blocks and slices add a multiple of 16 rows, which keeps the swizzle.
template <int D>
struct FragOffsets {
  int row[D / 16];
  int tlo[D / 32];
  int thi[D / 32];
  __device__ __forceinline__ explicit FragOffsets(int lane) {
    using T = BTile<D>;
    const int half = lane >> 5, rr = pi_row(lane & 31);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      row[kk] = rr * T::kRowB + (((2 * kk + half) ^ bswz<D>(rr)) & (T::kCh - 1)) * 16;
    const int g = lane >> 4, j = lane & 15;
    const int ra = 8 * (g >> 1) + (j >> 2);
    const int cc = 2 * (g & 1) + ((j & 3) >> 1), byte = 8 * (j & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + cc;
      tlo[db] = ra * T::kRowB + ((c ^ bswz<D>(ra)) & (T::kCh - 1)) * 16 + byte;
      thi[db] = (ra + 4) * T::kRowB + ((c ^ bswz<D>(ra + 4)) & (T::kCh - 1)) * 16 + byte;
    }
  }
};

// Order of the products inside one pipeline step: N1 score products and N2
// gradient products, N1 = R N2, as R score products then one gradient
// product, so consecutive products of one accumulator chain stay apart.
template <int N1, int N2>
__device__ constexpr bool op_is_grad(int i) {
  if constexpr (N1 == 0) {
    return true;
  } else if constexpr (N2 == 0) {
    return false;
  } else {
    constexpr int R = N1 / N2;
    return i % (R + 1) == R;
  }
}
template <int N1, int N2>
__device__ constexpr int op_index(int i) {
  if constexpr (N1 == 0 || N2 == 0) {
    return i;
  } else {
    constexpr int R = N1 / N2;
    return i % (R + 1) == R ? i / (R + 1) : (i / (R + 1)) * R + i % (R + 1);
  }
}

// Workgroup -> (batch*head unit, tile) over a grid of nbh * nt workgroups.
// Workgroup i runs on XCD i % 8.  order > 0: tile 0 has the most work,
// order < 0: the last tile has; then XCD x takes the units x, x + 8, ... and
// starts the longest tiles of all of them first.  order == 0: equal tiles,
// numbered so that each XCD holds whole units (their tiles share its L2).
__device__ __forceinline__ void bwd_unit(int nbh, int nt, int order, int& bh, int& t) {
  if (order != 0 && (nbh & 7) == 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3, hx = nbh >> 3;
    const int r = k / hx;
    bh = x + 8 * (k - r * hx);
    t = order > 0 ? r : nt - 1 - r;
  } else {
    const int id = xcd_contiguous(blockIdx.x, gridDim.x);
    bh = id / nt;
    t = id - bh * nt;
  }
}

// Compute units of the current device rounded down to a multiple of 8 (the
// grid of a persistent launch, one workgroup per CU); 0 if the query fails.
inline int bwd_slots() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n & ~7;
}

// Element masks without scalar compares: bit c of the word is set iff
// lo <= c <= hi (c = 16 (r / 8) + r % 8 in 0..31, the row or key offset of
// accumulator register r inside its block), and an element is kept by
// sign-extending its bit over the float.
__device__ __forceinline__ uint32_t mask_word(int lo, int hi) {
  const int l = max(lo, 0), h = min(hi, 31);
  const uint32_t below_h = h < 0 ? 0u : (2u << h) - 1u;   // bits 0..h
  const uint32_t below_l = l > 31 ? ~0u : (1u << l) - 1u;  // bits 0..l-1
  return below_h & ~below_l;
}
__device__ __forceinline__ float keep_bit(uint32_t m, int c, float x) {
  const uint32_t all = (uint32_t)((int)(m << (31 - c)) >> 31);
  return __uint_as_float(__float_as_uint(x) & all);
}

// Buffer descriptors and LDS slot of one tile's DMA.  Tiles past the last
// get descriptors of size 0: their loads fetch nothing and write zeros into a
// free ring slot, so every iteration issues the same number of loads and the
// waits use one constant count.
struct DmaTile {
  u32x4_t x, y, vec;
  uint32_t lds;  // LDS byte address of the ring slot
};

template <bool B>
using Bool = std::integral_constant<bool, B>;
template <int I>
using Int = std::integral_constant<int, I>;

// Owner fragments: rows [r0, r0 + 32) of a [rows][heads][D] tensor (head base
// g) as MFMA B operands, lane l32 = row, k-slots d = 16 kk + 8 h .. + 7; rows
// past n read as zeros.
template <int D>
__device__ __forceinline__ void load_owner(bf16x8_t (&f)[D / 16], const uint16_t* g, long long rs,
                                           int r0, int n, int lane) {
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const uint32_t nrec = (uint32_t)max(min(n - r0, kWaveRows), 0) * row_bytes;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g + (long long)max(r0, 0) * rs), 0, __builtin_amdgcn_readfirstlane(nrec), kRsrcWord3);
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const uint32_t off = (uint32_t)l32 * row_bytes + (uint32_t)(kk * 16 + half * 8) * 2;
    f[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

}  // namespace
}  // namespace fa
