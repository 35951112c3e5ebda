// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale Q K^T) V for
// an output gradient dO, recomputing the probabilities from the row
// log-sum-exp the forward pass emits instead of storing them -- the reason
// the forward keeps lse ("FlashAttention" (aiwiki.page), section "Training
// and computational complexity").  With P = exp(scale Q K^T - lse) (zero on
// masked pairs) the gradients are the chain rule through the softmax:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id (= rowsum(P o dP)),
//   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, no atomics (every output element has one writer), dq first:
//  * dq: one workgroup per (batch, head, 128 query rows); each wave owns 32
//    rows (Q and dO fragments in registers) while 64-key tiles of K and V
//    stream through the ring: S^T = K Q^T, dP^T = V dO^T, dS^T on the VALU,
//    then dQ^T += K^T dS^T.  It also reads its rows of O in the dO fragment
//    layout, forms D_i once the loop's first step (score products only) is
//    issued, and writes -D_i and -lse_i / scale of each row into the
//    workspace for the dkdv kernel.
//  * dkdv: one workgroup of 4 waves (one per SIMD) per (batch, head, 128
//    keys); each wave owns 32 keys and keeps their K and V fragments in
//    registers while 64-row tiles of Q, dO, -lse/scale, -D stream through a ring
//    of LDS slots.  -D and -lse / scale seed the dP and S accumulators, so
//    the products come out as dP - D and S - lse / scale and the VALU needs
//    one multiply less per element.  Per 32 query rows: S = Q K^T and
//    dP = dO V^T (keys in the lane, rows in the accumulator registers), P and
//    dS on the VALU, then dV^T += dO^T P and dK^T += Q^T dS with the tile
//    read transposed.
// Splitting dQ from dK/dV recomputes S and dP once more but needs neither
// atomics nor an fp32 dQ buffer, and the result is bit-reproducible.
//
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 before they enter a product.  The rows that form a
// score accumulator enter in pi order (bits 2 and 3 of the row index
// swapped), so each lane's accumulator registers are directly the k-slots of
// the next product's operand, and transposed operands come from
// ds_read_b64_tr_b16.
//
// Each wave runs a three-stage software pipeline over 32-row (32-key) blocks:
// one step issues the score products of block j+1 and the gradient products
// of block j-1 on the matrix pipe, interleaved, while the VALU turns the
// scores of block j into P and dS.  With one wave per SIMD this is what keeps
// the matrix pipe fed.
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
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

template <int D>
struct BTile {
  static constexpr int kCh = D / 8;                       // 16-byte chunks per row
  static constexpr int kRowB = D * 2;                     // bytes per row in LDS
  static constexpr int kBytes = kTile * kRowB;            // one tensor's tile
  static constexpr int kLoads = kBytes / 1024 / kBWaves;  // 1 KB DMA loads per wave per tensor
  static constexpr int kVec = kTile * 4;                  // one fp32 value per tile row
  static_assert(kBytes % (1024 * kBWaves) == 0, "tile must split evenly over the waves");
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
  char* lds;
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

// ---------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using T = BTile<D>;
  constexpr int kSlot = 2 * T::kBytes + 2 * T::kVec;  // Q tile, dO tile, -lse/scale, -D
  constexpr int kPer = 2 * T::kLoads + 1;             // DMA loads per wave per tile
  constexpr int kPieces = 3;                          // Q group, dO group, vector
  __shared__ __attribute__((aligned(1024))) char ring[kRing * kSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = a.heads, n_q = a.seqlen_q, n_k = a.seqlen_k, delta = n_k - n_q;
  const int W = a.window_left;
  const bool causal = a.causal != 0;
  const int nkt = ceil_div(n_k, kUnit);
  int bh, kt;
  bwd_unit(a.batch * H, nkt, causal ? 1 : (W >= 0 ? -1 : 0), bh, kt);
  const int h = bh % H, b = bh / H;
  const long long rs = (long long)H * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const int k0 = kt * kUnit, wk0 = k0 + wave * kWaveRows;
  const int key = wk0 + l32;  // this lane's key

  bf16x8_t kf[D / 16], vf[D / 16];
  load_owner<D>(kf, (const uint16_t*)a.k + ((long long)b * n_k * H + h) * D, rs, wk0, n_k, lane);
  load_owner<D>(vf, (const uint16_t*)a.v + ((long long)b * n_k * H + h) * D, rs, wk0, n_k, lane);

  f32x16_t dk[D / 32], dv[D / 32];  // dK^T, dV^T: [d][key], lane = key
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.0f;
      dv[db][r] = 0.0f;
    }

  // query rows that can see one of the workgroup's keys, in 64-row tiles
  int q_lo = 0, q_hi = n_q;
  if (causal) q_lo = max(q_lo, k0 - delta);
  if (W >= 0) q_hi = min(q_hi, k0 + kUnit - delta + W);
  const int t_lo = q_lo / kTile;
  const int nt = q_hi > q_lo ? ceil_div(q_hi, kTile) - t_lo : 0;

  const uint16_t* qg = (const uint16_t*)a.q + ((long long)b * n_q * H + h) * D;
  const uint16_t* gg = (const uint16_t*)a.dout + ((long long)b * n_q * H + h) * D;
  const float* nlg = a.ws_nl + ((long long)b * H + h) * n_q;
  const float* ndg = a.ws_nd + ((long long)b * H + h) * n_q;
  const float c2 = a.scale_log2;

  // DMA: wave w moves the 1 KB blocks 4w .. 4w + 3 of each tensor's tile;
  // lane l of block blk fills LDS position blk * 64 + l (row r, chunk slot p)
  // with logical chunk p ^ bswz(r).  xofs[i] is that memory offset minus the
  // instruction offset i * 1024 of block 4w + i (see dma_b128x4).
  static_assert(T::kLoads == 4 || T::kLoads == 2, "DMA grouping");
  uint32_t xofs[T::kLoads];
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int s = (wave * T::kLoads + i) * 64 + lane, r = s / T::kCh, p = s % T::kCh;
    xofs[i] = (uint32_t)r * row_bytes + (uint32_t)(((p ^ bswz<D>(r)) & (T::kCh - 1)) * 16) -
              (uint32_t)(i * 1024);
  }
  // this wave's blocks of one tensor's tile
  auto dma_group = [&](const u32x4_t& rsrc, uint32_t lds_base) {
    if constexpr (T::kLoads == 4) {
      dma_b128x4(rsrc, xofs[0], xofs[1], xofs[2], xofs[3], lds_base);
    } else {
      dma_b128(rsrc, xofs[0], lds_base);
      dma_b128(rsrc, xofs[1] + 1024, lds_base + 1024);
    }
  };
  auto slot = [&](int u) { return ring + (u & (kRing - 1)) * kSlot; };
  auto dma_setup = [&](int u) {
    DmaTile t;
    const int r0 = u < nt ? (t_lo + u) * kTile : 0;
    const uint32_t rows = u < nt ? (uint32_t)min(kTile, n_q - r0) : 0u;
    t.x = rsrc_of(qg + (long long)r0 * rs, rows * row_bytes);
    t.y = rsrc_of(gg + (long long)r0 * rs, rows * row_bytes);
    // waves 0, 2 load -lse/scale, waves 1, 3 load -D (the same values twice)
    t.vec = rsrc_of((wave & 1) ? ndg + r0 : nlg + r0, rows * 4);
    t.lds = slot(u);
    return t;
  };
  auto dma_piece = [&](const DmaTile& t, int k) {
    if (k < 2) {
      dma_group(k == 0 ? t.x : t.y, lds_addr(t.lds + k * T::kBytes + wave * T::kLoads * 1024));
    } else {
      dma_b32(t.vec, (uint32_t)lane * 4, lds_addr(t.lds + 2 * T::kBytes + (wave & 1) * T::kVec));
    }
  };

  const FragOffsets<D> fo(lane);
  f32x16_t sacc[2], dpacc[2];  // [block parity]: S and dP of one 32-row block
  bf16x8_t pf[2][2], sf[2][2];  // [block parity][16-row slice]: P and dS as B operands
  auto block_row0 = [&](int j) { return (t_lo + (j >> 1)) * kTile + kWaveRows * (j & 1); };
  auto block_masked = [&](int j) {
    const int r0 = block_row0(j);
    return (causal && wk0 + kWaveRows - 1 > r0 + delta) ||
           (W >= 0 && wk0 < r0 + kWaveRows - 1 + delta - W);
  };

  // one pipeline step: the score products of block j + 1 (M1), the gradient
  // products of block j - 1 (M2), P and dS of block j (VV), and with DMA the
  // loads of one later tile; PAR = j & 1.  The step is a sequence of chunks,
  // one per product: its operand reads kLook products ahead, the product, a
  // share of the probability work and of the loads.  sched_barrier keeps the
  // chunks in this order, so the vector work runs beside the matrix pipe
  // instead of after it (one wave per SIMD: nothing else would fill it).
  auto step = [&](auto M1, auto M2, auto VV, auto MASK, auto PAR, auto DMA, const DmaTile& dt,
                  int j) {
    constexpr bool kM1 = decltype(M1)::value, kM2 = decltype(M2)::value;
    constexpr bool kVV = decltype(VV)::value, kMask = decltype(MASK)::value;
    constexpr bool kDma = decltype(DMA)::value;
    constexpr int p = decltype(PAR)::value;
    constexpr int kN1 = kM1 ? 2 * (D / 16) : 0;
    constexpr int kN2 = kM2 ? 4 * (D / 32) : 0;
    constexpr int kN = kN1 + kN2;
    // block j + 1 and j - 1 have parity 1 - p: row block 1 - p of their tile
    const char* x1 = slot((j + 1) >> 1) + (1 - p) * kWaveRows * T::kRowB;
    const char* x2 = slot((j - 1) >> 1) + (1 - p) * kWaveRows * T::kRowB;

    auto fetch = [&](int i) -> bf16x8_t {
      const int o = op_index<kN1, kN2>(i);
      if (!op_is_grad<kN1, kN2>(i)) {
        return lds_row(x1 + (o & 1) * T::kBytes + fo.row[o >> 1]);
      } else {
        const int ks = o / (2 * (D / 32)), rem = o % (2 * (D / 32)), db = rem >> 1;
        const char* t = x2 + ((rem & 1) ? 0 : T::kBytes) + ks * 16 * T::kRowB;
        return lds_tr(t + fo.tlo[db], t + fo.thi[db]);
      }
    };
    // the score products of block j + 1 start from -lse/scale and -D of
    // their rows: register r of half h is row 16 (r / 8) + 8 h + r % 8
    f32x16_t nl_init, nd_init;
    if constexpr (kM1) {
      const char* vb = slot((j + 1) >> 1) + 2 * T::kBytes + (kWaveRows * (1 - p) + 8 * half) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int off = (q >> 1) * 64 + (q & 1) * 16;
        const f32x4_t x = lds_f4(vb + off), y = lds_f4(vb + T::kVec + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nl_init[4 * q + e] = x[e];
          nd_init[4 * q + e] = y[e];
        }
      }
    }
    auto product = [&](int i, const bf16x8_t& f) {
      const int o = op_index<kN1, kN2>(i);
      if (!op_is_grad<kN1, kN2>(i)) {
        const int kk = o >> 1;
        if (o & 1) {
          dpacc[1 - p] = mfma(f, vf[kk], kk == 0 ? nd_init : dpacc[1 - p]);
        } else {
          sacc[1 - p] = mfma(f, kf[kk], kk == 0 ? nl_init : sacc[1 - p]);
        }
      } else {
        const int ks = o / (2 * (D / 32)), rem = o % (2 * (D / 32)), db = rem >> 1;
        if (rem & 1) {
          dk[db] = mfma(f, sf[1 - p][ks], dk[db]);
        } else {
          dv[db] = mfma(f, pf[1 - p][ks], dv[db]);
        }
      }
    };

    // P and dS of block j from sacc = S - lse / scale, dpacc = dP - D, in
    // 32 pieces: pieces 0..15 exponentiate register q, pieces 16..31 form dS
    // of register q - 16 and pack pairs to bf16
    float ev[16], dsv[16];
    uint32_t pw[8], sw[8];
    auto vpiece = [&](int q) {
      if (q < 16) {
        ev[q] = exp2_hw(sacc[p][q] * c2);
        anchor(ev[q]);
      } else {
        const int t = q - 16;
        dsv[t] = ev[t] * dpacc[p][t];
        if (t & 1) {
          pw[t >> 1] = pack2(ev[t - 1], ev[t]);
          sw[t >> 1] = pack2(dsv[t - 1], dsv[t]);
          anchor(pw[t >> 1]);
          anchor(sw[t >> 1]);
        }
      }
    };
    // the same with the causal / window mask (pairs outside the band get 0),
    // for the few blocks that cross a mask edge
    auto probs_masked = [&]() {
      // key <= row + delta and key >= row + delta - W, row = r0 + 8 h + c
      const int w = key - delta - block_row0(j) - 8 * half;
      const uint32_t keep = mask_word(causal ? w : -kFar, W >= 0 ? w + W : kFar);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pv[8], dv8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int r = 8 * ks + t;
          const float e = keep_bit(keep, 16 * ks + t, exp2_hw(sacc[p][r] * c2));
          pv[t] = e;
          dv8[t] = e * dpacc[p][r];
        }
        pf[p][ks] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        sf[p][ks] = to_bf16x8(dv8[0], dv8[1], dv8[2], dv8[3], dv8[4], dv8[5], dv8[6], dv8[7]);
      }
    };

    if constexpr (kN > 0) {
      bf16x8_t fq[kLook + 1];
#pragma unroll
      for (int i = 0; i < kLook && i < kN; ++i) fq[i] = fetch(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kLook < kN) fq[(i + kLook) % (kLook + 1)] = fetch(i + kLook);
        product(i, fq[i % (kLook + 1)]);
        if constexpr (kVV) {
#pragma unroll
          for (int q = i * 32 / kN; q < (i + 1) * 32 / kN; ++q) vpiece(q);
        }
        if constexpr (kDma) {
#pragma unroll
          for (int k = 0; k < kPieces; ++k)
            if (k * kN / kPieces + kN / (2 * kPieces) == i) dma_piece(dt, k);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kVV) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pf[p][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});
        sf[p][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{sw[4 * ks], sw[4 * ks + 1], sw[4 * ks + 2], sw[4 * ks + 3]});
      }
      // blocks that cross a mask edge redo P and dS with the mask after the
      // step's products (their inputs stay intact until the next step)
      if constexpr (kMask) {
        if (block_masked(j)) probs_masked();
      }
    }
  };

  if (nt > 0) {
    constexpr Bool<true> y{};
    constexpr Bool<false> n{};
    {
      const DmaTile t0 = dma_setup(0), t1 = dma_setup(1);
#pragma unroll
      for (int k = 0; k < kPieces; ++k) dma_piece(t0, k);
#pragma unroll
      for (int k = 0; k < kPieces; ++k) dma_piece(t1, k);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));  // tile 0 has landed
    barrier();
    step(y, n, n, n, Int<1>{}, n, DmaTile{}, -1);
    step(y, n, y, y, Int<0>{}, y, dma_setup(2), 0);
    // iteration u: tile u lands, then P, dS of blocks 2u - 1 and 2u while the
    // loads of tile u + 2 go out (one loop: separate loops for masked and
    // unmasked blocks made the compiler spill the pipeline state to scratch)
    for (int u = 1; u < nt; ++u) {
      // tile u has landed once at most the loads of tile u + 1 are in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));
      barrier();  // tile u visible; every wave is done with tile u - 2
      step(y, y, y, y, Int<1>{}, y, dma_setup(u + 2), 2 * u - 1);
      step(y, y, y, y, Int<0>{}, n, DmaTile{}, 2 * u);
    }
    step(n, y, y, y, Int<1>{}, n, DmaTile{}, 2 * nt - 1);
    step(n, y, n, n, Int<0>{}, n, DmaTile{}, 2 * nt);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the size-0 loads of the last tiles
  }

  // lane holds d = 32 db + 8 (r/4) + 4 h + r%4 of its key
  if (key < n_k) {
    uint16_t* dkp = (uint16_t*)a.dk + (((long long)b * n_k + key) * H + h) * D;
    uint16_t* dvp = (uint16_t*)a.dv + (((long long)b * n_k + key) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        u32x2_t pk, pv;
        pk[0] = pack_bf16x2(a.scale * dk[db][g4 * 4 + 0], a.scale * dk[db][g4 * 4 + 1]);
        pk[1] = pack_bf16x2(a.scale * dk[db][g4 * 4 + 2], a.scale * dk[db][g4 * 4 + 3]);
        pv[0] = pack_bf16x2(dv[db][g4 * 4 + 0], dv[db][g4 * 4 + 1]);
        pv[1] = pack_bf16x2(dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3]);
        *(u32x2_t*)(dkp + d) = pk;
        *(u32x2_t*)(dvp + d) = pv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using T = BTile<D>;
  constexpr int kSlot = 2 * T::kBytes;  // K tile, V tile
  constexpr int kPer = 2 * T::kLoads;  // DMA loads per wave per tile
  constexpr int kPieces = 2;           // K group, V group
  __shared__ __attribute__((aligned(1024))) char ring[kRing * kSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = a.heads, n_q = a.seqlen_q, n_k = a.seqlen_k, delta = n_k - n_q;
  const int W = a.window_left;
  const bool causal = a.causal != 0;
  const int nqt = ceil_div(n_q, kUnit);
  int bh, qt;
  bwd_unit(a.batch * H, nqt, causal ? -1 : (W >= 0 ? 1 : 0), bh, qt);
  const int h = bh % H, b = bh / H;
  const long long rs = (long long)H * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const int q0 = qt * kUnit, wq0 = q0 + wave * kWaveRows;
  const int row = wq0 + l32;  // this lane's query row

  bf16x8_t qf[D / 16], gf[D / 16];
  load_owner<D>(qf, (const uint16_t*)a.q + ((long long)b * n_q * H + h) * D, rs, wq0, n_q, lane);
  load_owner<D>(gf, (const uint16_t*)a.dout + ((long long)b * n_q * H + h) * D, rs, wq0, n_q, lane);
  const bool row_live = row < n_q;
  // this lane's row of O, read in the fragment layout of dO (each half of the
  // wave holds one half of d), for D; used after the first pipeline step
  bf16x8_t of[D / 16];
  load_owner<D>(of, (const uint16_t*)a.o + ((long long)b * n_q * H + h) * D, rs, wq0, n_q, lane);
  const long long ridx = ((long long)b * H + h) * n_q + row;
  const float nl_row = row_live ? -a.lse[ridx] / a.scale : 0.0f;
  // exp2 argument offset (-lse * log2 e) and -D of this lane's row; rows past
  // n_q get probability 0
  float nlc = 0.0f, nd = 0.0f;
  // D = sum_d dO o O of the row; -D and -lse / scale (score units; +inf for
  // a row with no key) go into the workspace for the dkdv kernel
  auto row_terms = [&]() {
    float dsum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)of[kk][e], (float)gf[kk][e], dsum);
    dsum += __shfl_xor(dsum, 32);
    if (row_live && half == 0) {
      a.ws_nd[ridx] = -dsum;
      a.ws_nl[ridx] = nl_row;
    }
    nlc = row_live ? nl_row * a.scale_log2 : -__builtin_inff();
    nd = row_live ? -dsum : 0.0f;
  };

  f32x16_t dq[D / 32];  // dQ^T: [d][row], lane = row
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;

  // keys the workgroup's rows can see, in 64-key tiles
  const int q_last = min(q0 + kUnit, n_q) - 1;
  int k_lo = 0, k_hi = n_k;
  if (causal) k_hi = min(k_hi, q_last + delta + 1);
  if (W >= 0) k_lo = max(k_lo, q0 + delta - W);
  const int t_lo = k_lo / kTile;
  const int nt = k_hi > k_lo ? ceil_div(k_hi, kTile) - t_lo : 0;

  const uint16_t* kg = (const uint16_t*)a.k + ((long long)b * n_k * H + h) * D;
  const uint16_t* vg = (const uint16_t*)a.v + ((long long)b * n_k * H + h) * D;
  const float c2 = a.scale_log2;

  uint32_t xofs[T::kLoads];  // as in the dK, dV kernel
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int s = (wave * T::kLoads + i) * 64 + lane, r = s / T::kCh, p = s % T::kCh;
    xofs[i] = (uint32_t)r * row_bytes + (uint32_t)(((p ^ bswz<D>(r)) & (T::kCh - 1)) * 16) -
              (uint32_t)(i * 1024);
  }
  // this wave's blocks of one tensor's tile
  auto dma_group = [&](const u32x4_t& rsrc, uint32_t lds_base) {
    if constexpr (T::kLoads == 4) {
      dma_b128x4(rsrc, xofs[0], xofs[1], xofs[2], xofs[3], lds_base);
    } else {
      dma_b128(rsrc, xofs[0], lds_base);
      dma_b128(rsrc, xofs[1] + 1024, lds_base + 1024);
    }
  };
  auto slot = [&](int u) { return ring + (u & (kRing - 1)) * kSlot; };
  auto dma_setup = [&](int u) {
    DmaTile t;
    const int r0 = u < nt ? (t_lo + u) * kTile : 0;
    const uint32_t rows = u < nt ? (uint32_t)min(kTile, n_k - r0) : 0u;
    t.x = rsrc_of(kg + (long long)r0 * rs, rows * row_bytes);
    t.y = rsrc_of(vg + (long long)r0 * rs, rows * row_bytes);
    t.lds = slot(u);
    return t;
  };
  auto dma_piece = [&](const DmaTile& t, int k) {
    dma_group(k == 0 ? t.x : t.y, lds_addr(t.lds + k * T::kBytes + wave * T::kLoads * 1024));
  };

  const FragOffsets<D> fo(lane);
  f32x16_t sacc[2], dpacc[2];  // [block parity]: S^T and dP^T of one 32-key block
  bf16x8_t sf[2][2];            // [block parity][16-key slice]: dS^T as B operand
  auto block_key0 = [&](int j) { return (t_lo + (j >> 1)) * kTile + kWaveRows * (j & 1); };
  auto block_masked = [&](int j) {
    const int k0 = block_key0(j);
    return k0 + kWaveRows > n_k || (causal && k0 + kWaveRows - 1 > wq0 + delta) ||
           (W >= 0 && k0 < wq0 + kWaveRows - 1 + delta - W);
  };

  // one pipeline step, chunked as in the dK, dV kernel
  auto step = [&](auto M1, auto M2, auto VV, auto MASK, auto PAR, auto DMA, const DmaTile& dt,
                  int j) {
    constexpr bool kM1 = decltype(M1)::value, kM2 = decltype(M2)::value;
    constexpr bool kVV = decltype(VV)::value, kMask = decltype(MASK)::value;
    constexpr bool kDma = decltype(DMA)::value;
    constexpr int p = decltype(PAR)::value;
    constexpr int kN1 = kM1 ? 2 * (D / 16) : 0;
    constexpr int kN2 = kM2 ? 2 * (D / 32) : 0;
    constexpr int kN = kN1 + kN2;
    const char* x1 = slot((j + 1) >> 1) + (1 - p) * kWaveRows * T::kRowB;
    const char* x2 = slot((j - 1) >> 1) + (1 - p) * kWaveRows * T::kRowB;

    auto fetch = [&](int i) -> bf16x8_t {
      const int o = op_index<kN1, kN2>(i);
      if (!op_is_grad<kN1, kN2>(i)) {
        return lds_row(x1 + (o & 1) * T::kBytes + fo.row[o >> 1]);
      } else {
        const int ks = o / (D / 32), db = o % (D / 32);
        const char* t = x2 + ks * 16 * T::kRowB;
        return lds_tr(t + fo.tlo[db], t + fo.thi[db]);
      }
    };
    auto product = [&](int i, const bf16x8_t& f) {
      const int o = op_index<kN1, kN2>(i);
      if (!op_is_grad<kN1, kN2>(i)) {
        const int kk = o >> 1;
        if (o & 1) {
          dpacc[1 - p] = mfma(f, gf[kk], kk == 0 ? f32x16_t{} : dpacc[1 - p]);
        } else {
          sacc[1 - p] = mfma(f, qf[kk], kk == 0 ? f32x16_t{} : sacc[1 - p]);
        }
      } else {
        const int ks = o / (D / 32), db = o % (D / 32);
        dq[db] = mfma(f, sf[1 - p][ks], dq[db]);
      }
    };

    // dS^T of block j in 32 pieces: 0..15 exponentiate register q, 16..31
    // form dS of register q - 16 and pack pairs to bf16
    float ev[16], dsv[16];
    uint32_t sw[8];
    auto vpiece = [&](int q) {
      if (q < 16) {
        ev[q] = exp2_hw(fmaf(sacc[p][q], c2, nlc));
        anchor(ev[q]);
      } else {
        const int t = q - 16;
        dsv[t] = ev[t] * (dpacc[p][t] + nd);
        if (t & 1) {
          sw[t >> 1] = pack2(dsv[t - 1], dsv[t]);
          anchor(sw[t >> 1]);
        }
      }
    };
    // with the mask: keys outside the band or past n_k get 0
    auto probs_masked = [&]() {
      // key = k0 + 8 h + c: key < n_k, key <= row + delta, key >= row + delta - W
      const int base = block_key0(j) + 8 * half;
      const int v = row + delta - base;
      const uint32_t keep =
          mask_word(W >= 0 ? v - W : -kFar, causal ? min(n_k - 1 - base, v) : n_k - 1 - base);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float d8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int r = 8 * ks + t;
          const float e = keep_bit(keep, 16 * ks + t, exp2_hw(fmaf(sacc[p][r], c2, nlc)));
          d8[t] = e * (dpacc[p][r] + nd);
        }
        sf[p][ks] = to_bf16x8(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
      }
    };

    if constexpr (kN > 0) {
      bf16x8_t fq[kLook + 1];
#pragma unroll
      for (int i = 0; i < kLook && i < kN; ++i) fq[i] = fetch(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kLook < kN) fq[(i + kLook) % (kLook + 1)] = fetch(i + kLook);
        product(i, fq[i % (kLook + 1)]);
        if constexpr (kVV) {
#pragma unroll
          for (int q = i * 32 / kN; q < (i + 1) * 32 / kN; ++q) vpiece(q);
        }
        if constexpr (kDma) {
#pragma unroll
          for (int k = 0; k < kPieces; ++k)
            if (k * kN / kPieces + kN / (2 * kPieces) == i) dma_piece(dt, k);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kVV) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        sf[p][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{sw[4 * ks], sw[4 * ks + 1], sw[4 * ks + 2], sw[4 * ks + 3]});
      if constexpr (kMask) {
        if (block_masked(j)) probs_masked();
      }
    }
  };

  if (nt > 0) {
    constexpr Bool<true> y{};
    constexpr Bool<false> n{};
    {
      const DmaTile t0 = dma_setup(0), t1 = dma_setup(1);
#pragma unroll
      for (int k = 0; k < kPieces; ++k) dma_piece(t0, k);
#pragma unroll
      for (int k = 0; k < kPieces; ++k) dma_piece(t1, k);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));
    barrier();
    step(y, n, n, n, Int<1>{}, n, DmaTile{}, -1);
    // the first step needs no D; by now O has landed with tile 0
    row_terms();
    step(y, n, y, y, Int<0>{}, y, dma_setup(2), 0);
    for (int u = 1; u < nt; ++u) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));
      barrier();
      step(y, y, y, y, Int<1>{}, y, dma_setup(u + 2), 2 * u - 1);
      step(y, y, y, y, Int<0>{}, n, DmaTile{}, 2 * u);
    }
    step(n, y, y, y, Int<1>{}, n, DmaTile{}, 2 * nt - 1);
    step(n, y, n, n, Int<0>{}, n, DmaTile{}, 2 * nt);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    row_terms();
  }

  if (row_live) {
    uint16_t* qp = (uint16_t*)a.dq + (((long long)b * n_q + row) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        u32x2_t pq;
        pq[0] = pack_bf16x2(a.scale * dq[db][g4 * 4 + 0], a.scale * dq[db][g4 * 4 + 1]);
        pq[1] = pack_bf16x2(a.scale * dq[db][g4 * 4 + 2], a.scale * dq[db][g4 * 4 + 3]);
        *(u32x2_t*)(qp + d) = pq;
      }
  }
}

template <int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const long long g1 = (long long)a.batch * a.heads * ceil_div(a.seqlen_k, kUnit);
  const long long g2 = (long long)a.batch * a.heads * ceil_div(a.seqlen_q, kUnit);
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidValue;
  // dq first: it writes the per-row workspace values that dkdv reads
  if (g2 > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)g2), dim3(kBThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g1 > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)g1), dim3(kBThreads), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_bwd_t<128>(a, stream);
  if (d == 64) return launch_bwd_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
