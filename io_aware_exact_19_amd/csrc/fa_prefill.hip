// Tiled attention forward (prefill) for gfx950.
//
// One workgroup owns a tile of query rows of one (sequence, head) and streams
// that head's K/V tiles through LDS, keeping per-row running statistics
// (maximum m, exponential sum l) and an unnormalised output accumulator, so
// the score and probability matrices never leave the chip.  This is the
// tiled evaluation with online normalisation of "FlashAttention"
// (aiwiki.page), section "Tiling and online normalisation" (update equations
// for m', l', u' and the final division u / l), with the loop structure of
// the flowchart in "How FlashAttention accelerates Transformer attention with
// IO-aware tiling" (wiblog.cn), section "IO-aware tiling": load a Q block,
// then for each K/V block compute local scores, update row max and
// normaliser, accumulate the output; write the output once at the end.
//
// gfx950 mapping (not from the pages).  Common to both bf16 kernels:
//  * Each wave owns 32 whole query rows, so row statistics need no LDS
//    traffic.  Scores are produced transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16: each lane then holds the keys of a single
//    query row, so the row max/sum is in-lane plus one lane-half swap, and
//    the output accumulator O^T = V^T P^T gives each lane a single query row
//    as well.
//  * K rows enter the score product in a permuted order so that a lane's
//    probabilities are already the k-slots the P V product wants: no data
//    movement between the two products.
//  * The softmax works in base 2 with log2(e) folded into the scale
//    (v_exp_f32); the reference max is lazy (below) and the division by the
//    row sum happens once per row at the end.
//  * K and V tiles of 64 keys go from HBM straight into LDS (buffer loads
//    with the LDS destination, no register staging; rows past the sequence
//    end come back as zeros from the descriptor bound).  V stays row-major in
//    LDS and the P V operand is read with the transposing LDS read
//    (ds_read_b64_tr_b16).  K and V use different 16-byte-chunk swizzles,
//    each free of bank conflicts for its own read pattern.
//  * Fully masked K/V tiles (causal, sliding window) are never loaded;
//    element masks run only on tiles that cross a mask boundary.
//
// d = 128: ping-pong kernel.  8 waves (256 query rows) per workgroup, two per
//    SIMD.  The waves form two groups, one wave of each on every SIMD; work
//    alternates between a matrix block (P V of the previous tile and S of the
//    current one: 32 MFMAs per wave, operands streamed from LDS a few
//    products ahead) and a vector block (mask, online-softmax update, bf16
//    probabilities).  Group 1 runs half a step behind group 0 and a
//    workgroup barrier between the blocks keeps that offset, so on every
//    SIMD one wave's matrix block runs next to the other wave's softmax; the
//    wave in its matrix block raises its issue priority.  Tiles stream
//    through a ring of four LDS slots two tiles ahead of use; the loads are
//    queued with inline assembly so that the only waits for them are the
//    explicit ones before each step's barrier.  Plain dense launches are
//    persistent: one workgroup per CU walks several query tiles, and each
//    tile's last landing barrier queues the next tile's first K/V tiles and
//    Q fragments, so their latency runs under the last P V block and the
//    output stores.
// d = 64: four-wave kernel.  4 waves (128 query rows) per workgroup, two
//    workgroups per CU, double-buffered tiles, one barrier per tile.  At
//    d = 64 the softmax work per tile is as large as at d = 128 while the
//    matrix work halves, so the ping-pong split does not pay there.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBC = 64;  // keys per K/V tile

// bf16 ping-pong kernel (d = 128)
constexpr int kWaves = 8;                // two groups of 4, one wave of each per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * 32;         // query rows per workgroup

// bf16 four-wave kernel (d = 64)
constexpr int kQWaves = 4;
constexpr int kQThreads = kQWaves * 64;
constexpr int kQRows = kQWaves * 32;

// fp32 kernel geometry
constexpr int kWaves32 = 4;
constexpr int kThreads32 = kWaves32 * 64;
constexpr int kBR32 = kWaves32 * 32;
constexpr int kBC32 = 32;

// Row order of a 32-key block in the score product: bits 2 and 3 of the row
// index swapped.  Accumulator register r of lane-half h then holds key
// 16*(r/8) + 8*h + r%8 of the block.
__device__ __forceinline__ int pi_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Per-workgroup work item.
struct Work {
  int h;
  int qt;                 // query tile index within the sequence
  int n_q, n_k;           // sequence lengths
  long long q_row0;       // first packed row of the sequence in q/o
  long long k_row0;       // first packed row of the sequence in k/v
  long long lse_base;     // lse offset of the sequence's row 0 for head h
};

// Sequence with the r-th longest KV cache (ties: lower index first), for at
// most 64 sequences; the same value in every lane
__device__ __forceinline__ int kv_seq_by_rank(const FwdArgs& a, int r) {
  const int lane = threadIdx.x & 63;
  const int len = lane < a.batch ? min(max(a.seqlens_k[lane], 0), a.kv_rows) : -1;
  int rank = 0;
  for (int j = 0; j < a.batch; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const unsigned long long m = __builtin_amdgcn_ballot_w64(lane < a.batch && rank == r);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(m));
}

// KV: a KV-cache launch (its own kernel instantiation, so that the other
// launches carry none of this code)
template <bool KV>
__device__ __forceinline__ void dense_work(const FwdArgs& a, int nqt, Work& w, int item, int n_items) {
  const int nbh = a.batch * a.heads;
  int bh = 0, t = 0;  // t: rank of the tile in start order, 0 = started first
  bool ordered = false;
  if constexpr (KV) {
    if ((a.causal || a.window_left >= 0) && a.heads % 8 == 0 && a.batch <= 64) {
      // KV caches of different lengths: XCD x (workgroup i runs on XCD i %
      // 8) takes heads x, x + 8, ... of every sequence and starts them
      // longest cache first, the tiles of one (sequence, head) next to each
      // other so that they run together and read its keys once through the
      // XCD's L2
      const int x = item & 7, k = item >> 3, upx = a.heads >> 3;
      const int j = k / nqt;
      t = k - j * nqt;
      const int r = j / upx, mh = j - r * upx;
      bh = kv_seq_by_rank(a, r) * a.heads + x + 8 * mh;
      ordered = true;
    }
  }
  if (ordered) {
  } else if ((a.causal || a.window_left >= 0) && nbh % 8 == 0) {
    // Tiles differ in length.  Workgroup i goes to XCD i % 8, which starts
    // its workgroups in order as CUs free up: give XCD x the (batch, head)
    // units x, x + 8, x + 16, ... (a share of every sequence, which matters
    // when sequences differ in length) and let it start all their tiles
    // longest first, so the short tiles fill in behind the long ones
    // (longest-processing-time order); each unit's tiles stay on one XCD and
    // share its L2.
    const int x = item & 7, k = item >> 3, hx = nbh >> 3;
    t = k / hx;
    bh = x + 8 * (k - t * hx);
  } else {
    const int id = xcd_contiguous(item, n_items);
    bh = id / nqt;
    t = id - bh * nqt;
  }
  const int b = bh / a.heads;
  w.h = bh - b * a.heads;
  // causal: later tiles see more keys; a left window without the causal
  // bound: earlier tiles see more keys
  w.qt = a.causal || a.window_left < 0 ? nqt - 1 - t : t;
  w.n_q = a.seqlen_q;
  w.q_row0 = (long long)b * a.seqlen_q;
  w.lse_base = ((long long)b * a.heads + w.h) * a.seqlen_q;
  if (a.seqlens_k != nullptr) {
    // KV cache: the sequence's keys are the first seqlens_k[b] rows of its
    // kv_rows-row block (clamped to the block); the queries are its last
    // seqlen_q positions (bottom-right alignment)
    w.n_k = min(max(a.seqlens_k[b], 0), a.kv_rows);
    w.k_row0 = (long long)b * a.kv_rows;
  } else {
    w.n_k = a.seqlen_k;
    w.k_row0 = (long long)b * a.seqlen_k;
  }
}

// Inclusive prefix sum across the 64 lanes of a wave on the DPP network: row
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
// rows 0 and 2 added to rows 1 and 3 and the last lane of row 1 to rows 2
// and 3 (row broadcasts).  Six adds, no LDS round trips.
__device__ __forceinline__ int wave_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Variable-length scheduler: every wave reads the per-sequence offsets from
// cu_seqlens_q/k (64 sequences per round, all four bounds of a sequence in
// flight together; no host round trip), counts each sequence's query tiles
// ceil(len_q / rows), drops the workgroups past the live total, renumbers the
// rest XCD-contiguously and finds its (head, sequence, tile).  Head-major
// order keeps the tiles of one (sequence, head) on one XCD; the hardware
// starts a new workgroup whenever one ends, so the order is also the order
// in which work is handed out.  With at most 64 sequences the offsets are read
// once and the lookup works on registers.
//
// Order within a head: with a causal mask and a left window of W keys, a
// query tile t (rows beginning at t * rows) needs keys from t * rows + delta
// - W on, so every tile from kSat = ceil((W + 1) / rows) on costs the same
// (about W + rows keys) while the first kSat tiles of a sequence ramp up
// from one key tile.  The head's items run as: the full-cost tiles of every
// sequence (sequence order, latest tile first, so neighbouring items share
// key tiles), then the short ramp tiles from the longest down (tile kSat - 1
// of every sequence, then kSat - 2, ...), so the last items handed out are
// the shortest and workgroups finish close together.  Without such a window
// the order is sequence by sequence, latest tile first.
__device__ bool varlen_work(const FwdArgs& a, int rows, int lane, Work& w) {
  const int nseq = a.batch;
  // ramp length in tiles (0: no reordering)
  const int ksat = a.causal && a.window_left >= 0 ? ceil_div(a.window_left + 1, rows) : 0;
  int cq0 = 0, cq1 = 0, ck0 = 0, ck1 = 0, nt = 0, nl = 0, inc = 0;
  auto load_chunk = [&](int s0) {
    const int s = s0 + lane;
    const bool ok = s < nseq;
    cq0 = ok ? a.cu_q[s] : 0;
    cq1 = ok ? a.cu_q[s + 1] : 0;
    ck0 = ok ? a.cu_k[s] : 0;
    ck1 = ok ? a.cu_k[s + 1] : 0;
    nt = ok ? ceil_div(max(cq1 - cq0, 0), rows) : 0;
    nl = ksat > 0 ? max(nt - ksat, 0) : nt;  // full-cost tiles, handed out first
    inc = wave_scan_dpp(nl);
  };
  int total = 0, total_long = 0, total_q = 0;
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    load_chunk(s0);
    total_long += __builtin_amdgcn_readlane(inc, 63);
    total += __builtin_amdgcn_readlane(wave_scan_dpp(nt), 63);
    if (s0 + 64 >= nseq) total_q = __builtin_amdgcn_readlane(cq1, nseq - 1 - s0);
  }
  // uniform by construction; say so, so that the work decode stays in scalar
  // registers (else the tile loop and the buffer descriptors built from it
  // would be treated as divergent)
  total = __builtin_amdgcn_readfirstlane(total);
  total_long = __builtin_amdgcn_readfirstlane(total_long);
  const long long live = (long long)total * a.heads;
  if ((long long)blockIdx.x >= live) return false;
  const int id = xcd_contiguous(blockIdx.x, (int)live);
  w.h = id / total;
  const int g = id - w.h * total;
  int src = -1, qt = 0;
  if (g < total_long) {
    // full-cost tile number t of its sequence, latest first
    int base = 0;
    for (int s0 = 0; s0 < nseq; s0 += 64) {
      if (nseq > 64) load_chunk(s0);  // else chunk 0 is still in registers
      const int end = base + inc, beg = end - nl;
      const unsigned long long hit = __ballot(s0 + lane < nseq && g >= beg && g < end);
      if (hit) {
        src = __builtin_ctzll(hit);
        qt = __builtin_amdgcn_readlane(nt, src) - 1 - (g - __builtin_amdgcn_readlane(beg, src));
        break;
      }
      base += __builtin_amdgcn_readlane(inc, 63);
    }
  } else {
    // ramp tiles: level lvl = ksat - 1, ksat - 2, ..., 0 holds tile lvl of
    // every sequence with more than lvl tiles, in sequence order (a level no
    // sequence reaches holds none)
    int r = g - total_long;
    for (int lvl = ksat - 1; lvl >= 0 && src < 0; --lvl) {
      for (int s0 = 0; s0 < nseq; s0 += 64) {
        if (nseq > 64) load_chunk(s0);  // else chunk 0 is still in registers
        unsigned long long has = __ballot(s0 + lane < nseq && nt > lvl);
        const int cnt = __builtin_popcountll(has);
        if (r < cnt) {
          for (int k = r; k > 0; --k) has &= has - 1;  // drop the r lowest owners
          src = __builtin_ctzll(has);
          qt = lvl;
          break;
        }
        r -= cnt;
      }
    }
  }
  if (src < 0) return false;
  const int q0 = __builtin_amdgcn_readlane(cq0, src), q1 = __builtin_amdgcn_readlane(cq1, src);
  const int k0 = __builtin_amdgcn_readlane(ck0, src), k1 = __builtin_amdgcn_readlane(ck1, src);
  w.qt = qt;
  w.n_q = q1 - q0;
  w.n_k = max(k1 - k0, 0);
  w.q_row0 = q0;
  w.k_row0 = k0;
  w.lse_base = (long long)w.h * total_q + q0;
  return true;
}

// One K or V tile in LDS: kBC rows x D bf16, row-major as in HBM, with the
// 16-byte chunks of each row permuted (swizzled) per row.
template <int D, int THREADS>
struct BfTile {
  static constexpr int kKch = D / 8;                     // 16-byte chunks per row
  static constexpr int kBytes = kBC * D * 2;             // one tile
  static constexpr int kLoads = kBytes / 16 / THREADS;   // 16-byte DMA loads per thread per tile
  static_assert(kBytes % (16 * THREADS) == 0, "tile must split evenly over the threads");
};

// K tiles: chunk c of row r at c ^ tile_swz(r).  The score product's
// 16-lane groups read one chunk of 16 rows, which must land on 16 distinct
// 16-byte bank groups of a 256-byte bank line.  At d = 128 a row is one
// bank line, so the 16 swizzles must differ; at d = 64 two rows share a
// line (the row's parity picks its half), so the 8 rows of each parity need
// distinct swizzles in 0..7: row bits 1..3.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 64) {
    return (r >> 1) & 7;
  } else {
    return (r & 3) | ((r >> 1) & 4) | ((r << 1) & 8);
  }
}

template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + ((c ^ tile_swz<D>(r)) & (D / 8 - 1)) * 16;
}

// V tiles are read only through the transposing read, whose 16-lane groups
// touch 4 consecutive rows x 2 adjacent chunks: spread those rows over
// distinct bank groups (bits 1-3 of the chunk index).
__device__ __forceinline__ int vtile_swz(int r) {
  return (0xAC60 >> ((r & 3) * 4)) & 15;  // {0, 6, 12, 10}
}

template <int D>
__device__ __forceinline__ int vtile_off(int r, int c) {
  return r * (D * 2) + ((c ^ vtile_swz(r)) & (D / 8 - 1)) * 16;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// Raw buffer descriptor over [base, base + bytes).
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcWord3;
  return r;
}

// 16 bytes per lane from the buffer (byte offset voff) straight into LDS at
// lds_base + 16 * lane; offsets past the descriptor's size read as zeros.
// Issued as inline assembly so that the compiler does not track it: every
// wait for these loads is an explicit vmcnt wait before a barrier, and LDS
// reads of other ring slots never wait for them.  M0 (the LDS destination)
// is saved and restored around the load.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc_in, uint32_t voff, uint32_t lds_base) {
  u32x4_t rsrc;  // uniform by construction; keep it in scalar registers
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc_in[i]);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}

// A pointer every lane holds the same value of, moved to scalar registers, so
// that buffer descriptors built from it are known to be uniform (otherwise
// the compiler wraps each buffer access in a loop over the distinct values).
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)p);
}

// Lane-half exchange on the VALU: {r0, r1} = {x[lane], x[lane ^ 32]}.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lazy reference maximum: the output u / l does not depend on which reference
// value the exponentials are taken against, so a tile is exponentiated
// against the current reference and kept when each lane's probabilities sum
// to at most this bound; probabilities then stay <= 2^16, far from fp32 /
// bf16 overflow.
constexpr float kLazyBound = 65536.0f;

// Reductions over N x 16 values with independent partial results (short
// dependency chains: the vector block runs while its SIMD's other wave
// keeps the matrix pipe busy, so its latency is not hidden by another wave).
template <int N>
__device__ __forceinline__ float tree_sum(const float (&v)[N][16]) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = v[0][2 * i] + v[0][2 * i + 1];
#pragma unroll
  for (int n = 1; n < N; ++n)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] += v[n][2 * i] + v[n][2 * i + 1];
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}
template <int N>
__device__ __forceinline__ float tree_max(const f32x16_t (&v)[N]) {
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = fmaxf(fmaxf(v[0][4 * i], v[0][4 * i + 1]), fmaxf(v[0][4 * i + 2], v[0][4 * i + 3]));
#pragma unroll
  for (int n = 1; n < N; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = fmaxf(a[i], fmaxf(fmaxf(v[n][4 * i], v[n][4 * i + 1]), fmaxf(v[n][4 * i + 2], v[n][4 * i + 3])));
  return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
}

// Maximum of N x 16 values with three-input maxima (v_max3_f32, two new
// values per instruction) in four independent chains.
template <int N>
__device__ __forceinline__ float tree_max3(const f32x16_t (&v)[N]) {
  float a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = fmaxf(v[0][4 * c], v[0][4 * c + 1]);
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i0 = n == 0 ? 4 * c + 2 : 4 * c;
      a[c] = __builtin_fmaxf(__builtin_fmaxf(a[c], v[n][i0]), v[n][i0 + 1]);
      if (n > 0) a[c] = __builtin_fmaxf(__builtin_fmaxf(a[c], v[n][4 * c + 2]), v[n][4 * c + 3]);
    }
  return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
}

// acc + the sum of 8 bf16 values (dot products with (1, 1) in fp32).  The
// pairs are extracted as bf16x2 halves of the vector itself.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum_rounded_pairs(const bf16x8_t& v, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

// s_waitcnt immediates: wait until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier that is also a compiler memory barrier but carries no
// implicit wait: the tile loads that must have landed are waited for
// explicitly (vmcnt) before it, so loads of later tiles stay in flight.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int D, bool VARLEN, bool KV>
__device__ __forceinline__ void fwd_bf16_body(const FwdArgs& a) {
  using T = BfTile<D, kThreads>;
  // ring of 4 tile slots; slot s holds K at s * 2 * kBytes and V right after
  __shared__ __attribute__((aligned(1024))) char ring[4 * 2 * T::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;                 // 0: matrix block first; 1: half a tile later
  const int rblk = 2 * (wave & 3) + group;     // the two waves of a SIMD own adjacent rows
  const int half = lane >> 5, l32 = lane & 31;
  const int lg = lane >> 4, j16 = lane & 15;

  const long long rs = (long long)a.heads * D;  // elements between consecutive rows
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2;

  // Work items (query tiles of one (sequence, head)).  Dense launches may be
  // persistent: workgroup b takes items b, G + b', 2 G + b, ... (G = grid
  // size, a multiple of 8 when there is more than one round, so every item
  // of a workgroup belongs to its XCD); odd rounds take the mirror image b'
  // of b within its XCD, which pairs long causal tiles with short ones.
  // Varlen and single-round launches run one item per workgroup.
  const int nqt = ceil_div(a.seqlen_q, kBR);
  const int n_items = VARLEN ? (int)gridDim.x : a.batch * a.heads * nqt;
  auto item_id = [&](int r) {
    const int G = gridDim.x, b = blockIdx.x;
    const int bm = (r & 1) && (G & 7) == 0 ? (((G >> 3) - 1 - (b >> 3)) << 3) + (b & 7) : b;
    return r * G + bm;
  };

  // per-item state
  struct Item {
    const uint16_t* qg;
    const uint16_t* kg;
    const uint16_t* vg;
    uint16_t* og;
    long long lse_base;
    int n_q, n_k, t_lo, nt, wq0, wq_last, w_lo, w_hi;
    bool wave_live;
    int seg0, seg_end;
    u32x4_t rk, rv;
  };
  auto make_item = [&](int id, Item& it) -> bool {
    Work w;
    if constexpr (VARLEN) {
      if (!varlen_work(a, kBR, lane, w)) return false;
    } else {
      if (id >= n_items) return false;
      dense_work<KV>(a, nqt, w, id, n_items);
    }
    it.qg = (const uint16_t*)a.q + (w.q_row0 * a.heads + w.h) * D;
    it.kg = (const uint16_t*)a.k + (w.k_row0 * a.heads + w.h) * D;
    it.vg = (const uint16_t*)a.v + (w.k_row0 * a.heads + w.h) * D;
    it.og = (uint16_t*)a.o + (w.q_row0 * a.heads + w.h) * D;
    it.lse_base = w.lse_base;
    it.n_q = w.n_q;
    it.n_k = w.n_k;
    const int delta = w.n_k - w.n_q;
    const int q0 = w.qt * kBR;
    const int q_last = min(q0 + kBR, w.n_q) - 1;
    // K/V tiles the workgroup needs (fully masked ones are skipped)
    int kv_lo = 0, kv_hi = w.n_k;
    if (causal) kv_hi = min(kv_hi, q_last + delta + 1);
    if (W >= 0) kv_lo = max(kv_lo, q0 + delta - W);
    it.t_lo = kv_lo / kBC;
    it.nt = kv_hi > kv_lo ? ceil_div(kv_hi, kBC) - it.t_lo : 0;
    // this wave's rows and key range
    it.wq0 = q0 + rblk * 32;
    it.wave_live = it.wq0 < w.n_q;
    it.wq_last = min(it.wq0 + 31, w.n_q - 1);
    it.w_lo = 0;
    it.w_hi = w.n_k;
    if (causal) it.w_hi = min(it.w_hi, it.wq_last + delta + 1);
    if (W >= 0) it.w_lo = max(it.w_lo, it.wq0 + delta - W);
    it.seg0 = 0;
    it.seg_end = -1;
    it.rk = buffer_rsrc(it.kg, 0);
    it.rv = buffer_rsrc(it.vg, 0);
    return true;
  };

  // K/V streaming: one buffer descriptor per tensor covers a window of
  // seg_rows key rows from seg0 (32-bit offsets); rows past the sequence end
  // fall outside it and read as zeros.  The window moves only when a tile
  // would cross its end, which never happens below 2^32 bytes of keys.
  uint32_t kofs[T::kLoads], vofs[T::kLoads];
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int slot = (i * kWaves + wave) * 64 + lane;
    const int r = slot / T::kKch;
    const int ck = ((slot % T::kKch) ^ tile_swz<D>(r)) & (T::kKch - 1);
    const int cv = ((slot % T::kKch) ^ vtile_swz(r)) & (T::kKch - 1);
    kofs[i] = (uint32_t)r * row_bytes + (uint32_t)ck * 16;
    vofs[i] = (uint32_t)r * row_bytes + (uint32_t)cv * 16;
  }
  // ring slot of tile g, counted over all items of the workgroup
  const uint32_t ring_lds = lds_addr(ring);
  auto kslot = [&](int g) { return ring + (g & 3) * 2 * T::kBytes; };
  auto vslot = [&](int g) { return ring + (g & 3) * 2 * T::kBytes + T::kBytes; };
  // queue the DMA of tile j (relative to the item's t_lo) into slot g
  auto issue = [&](Item& it, int j, int g) {
    const int k0 = (it.t_lo + j) * kBC;
    if (k0 + kBC > it.seg_end) {
      it.seg0 = k0;
      it.seg_end = k0 + a.seg_rows;
      const uint32_t nrec = (uint32_t)min(it.n_k - k0, a.seg_rows) * row_bytes;
      it.rk = buffer_rsrc(it.kg + (long long)k0 * rs, nrec);
      it.rv = buffer_rsrc(it.vg + (long long)k0 * rs, nrec);
    }
    const uint32_t base = (uint32_t)(k0 - it.seg0) * row_bytes;
    // LDS byte address of the slot as an integer (no pointer casts on this
    // path: a cast of a ring pointer chosen at run time back to the LDS
    // address space can leave an aperture compare the code generator rejects)
    const uint32_t kdst = ring_lds + (uint32_t)(g & 3) * 2 * T::kBytes;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
      const uint32_t blk = (uint32_t)(i * kWaves + wave) * 1024;
      dma16(it.rk, base + kofs[i], kdst + blk);
      dma16(it.rv, base + vofs[i], kdst + T::kBytes + blk);
    }
  };
  // Q^T operand fragments: lane holds Q[qi][kk*16 + half*8 .. +8]; rows past
  // the sequence read as zeros through the descriptor bound
  bf16x8_t qf[D / 16];
  auto load_q = [&](const Item& it) {
    const uint32_t nrec =
        __builtin_amdgcn_readfirstlane((uint32_t)max(min(it.n_q - it.wq0, 32), 0) * row_bytes);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(it.qg + (long long)it.wq0 * rs), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
          rq, (uint32_t)l32 * row_bytes + (uint32_t)(kk * 16 + half * 8) * 2, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  };
  // first two tiles and the Q fragments of an item, tiles into slots g, g + 1
  auto start_loads = [&](Item& it, int g) {
    if (it.nt > 0) {
      issue(it, 0, g);
      if (it.nt > 1) issue(it, 1, g + 1);
    }
    load_q(it);
  };

  int r_item = 0;
  {
    Item first;
    if (!make_item(item_id(0), first)) return;
    start_loads(first, 0);
  }
  int gbase = 0;  // ring index of the current item's tile 0

  // per-row state of an item: the O accumulator u, the reference max m
  // (base-2 scaled), and this lane-half's partial exp-sums, unrounded (l, for
  // lse) and over the bf16-rounded probabilities (for O)
  f32x16_t oacc[D / 32];
  float m_run, l_run, lr_run;
  auto init_state = [&]() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    m_run = kNegInf;
    l_run = 0.0f;
    lr_run = 0.0f;
  };
  // O = u / l (one division per row, l over the rounded probabilities),
  // lse = ln 2 * (m + log2 l) (l over the unrounded ones)
  auto epilogue = [&](uint16_t* og_, int qi_, int n_q_, long long lse_base_) {
    const float l_tot = sum_halves(l_run);
    const float lr_tot = sum_halves(lr_run);
    if (qi_ < n_q_) {
      const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
      uint16_t* op = og_ + (long long)qi_ * rs;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + half * 4;
          u32x2_t pr;
          pr[0] = pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
          pr[1] = pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
          *(u32x2_t*)(op + d) = pr;
        }
      if (a.lse != nullptr && half == 0)
        a.lse[lse_base_ + qi_] = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : kNegInf;
    }
  };
  // Group 1 ends an item half a step after group 0.  Its epilogue is held
  // over into the next item and run after that item's first landing barrier,
  // while group 0 computes the first scores (group 1 would wait there
  // anyway), so group 0 no longer waits for it; the state stays in registers.
  bool pend = false;
  uint16_t* p_og = nullptr;
  int p_qi = 0, p_nq = 0;
  long long p_lse = 0;
  for (;;) {
  // the item's state is derived again here (its loads were queued earlier;
  // the K/V descriptor window restarts at the first tile queued from here)
  Item cur;
  make_item(item_id(r_item), cur);
  uint16_t* const og = cur.og;
  const int n_q = cur.n_q, n_k = cur.n_k, delta = n_k - n_q;
  const int t_lo = cur.t_lo, nt = cur.nt;
  const int wq0 = cur.wq0, wq_last = cur.wq_last, w_lo = cur.w_lo, w_hi = cur.w_hi;
  const bool wave_live = cur.wave_live;
  const int qi = wq0 + l32;  // this lane's query row
  // Q and the first two tiles are in flight together (with group 0's output
  // stores of the previous item); the wait covers all
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));


  // per-lane parts of the LDS operand addresses
  // K rows enter in pi order (see pi_row); sub-block kb adds 32 rows.  The
  // chunk (2 kk + half) ^ tile_swz(r) splits into the fixed low bit and
  // (kk ^ y) in the upper bits, so fragment kk sits at k_base + ((kk << 5) ^ k_y).
  int k_base, k_y;
  {
    const int r = pi_row(l32), sw = tile_swz<D>(r);
    k_base = r * D * 2 + ((half ^ sw) & 1) * 16;
    k_y = ((sw >> 1) & (D / 16 - 1)) << 5;
  }
  // V^T fragments through the transposing read: lane j of 16-lane group g
  // addresses row (ks*16 + 8*(g/2) + 4*u + j/4), dims db*32 + 16*(g%2) + 4*(j%4)
  int v_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int r = 8 * (lg >> 1) + (j16 >> 2);
    const int d = db * 32 + 16 * (lg & 1) + 4 * (j16 & 3);
    v_off[db] = vtile_off<D>(r, d >> 3) + (d & 7) * 2;
  }

  f32x16_t sacc[kBC / 32];    // scores of the current tile (matrix block -> vector block)
  bf16x8_t pf[kBC / 16];      // probabilities of the previous tile (vector block -> matrix block)

  auto live = [&](int j) {
    const int k0 = (t_lo + j) * kBC;
    return wave_live && j >= 0 && j < nt && k0 < w_hi && k0 + kBC > w_lo;
  };

  constexpr int kPV = (kBC / 16) * (D / 32);  // P V products per tile
  constexpr int kS = (D / 16) * (kBC / 32);   // score products per tile
  constexpr int kLook = 4;
  // issue order of the matrix block: P V and score products alternate, so
  // each accumulator chain has several independent products between its
  // own (the score chains are only kBC/32 deep)
  auto op = [&](int i) { return (i & 1) ? kPV + (i >> 1) : (i >> 1); };
  static_assert(kPV == kS, "alternating order needs equal product counts");
  // operand of product i: V^T fragment (i < kPV) or K fragment
  auto fetch = [&](int i, const char* kb_lds, const char* vp_lds) {
    if (i < kPV) {
      const int ks = i / (D / 32), db = i % (D / 32);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)(vp_lds + v_off[db] + ks * 16 * D * 2));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)(vp_lds + v_off[db] + ks * 16 * D * 2 + 4 * D * 2));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int kk = (i - kPV) / (kBC / 32), kb = (i - kPV) % (kBC / 32);
    return *(const bf16x8_t*)(kb_lds + (((kk << 5) ^ k_y) + k_base) + kb * 32 * D * 2);
  };
  auto product = [&](int i, const bf16x8_t& f) {
    if (i < kPV) {
      const int ks = i / (D / 32), db = i % (D / 32);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[ks], oacc[db], 0, 0, 0);
    } else {
      const int kk = (i - kPV) / (kBC / 32), kb = (i - kPV) % (kBC / 32);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[kk], sacc[kb], 0, 0, 0);
    }
  };
  // matrix block: P V of the previous tile (probabilities are zero when that
  // tile was not live for this wave) and S of tile j; the operand fragments
  // stream through a queue kLook products ahead of their use
  auto mblock = [&](const char* kb_lds, const char* vp_lds) {
    __builtin_amdgcn_s_setprio(2);  // the matrix stream wins issue arbitration on its SIMD
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
    bf16x8_t fq[kLook + 1];
#pragma unroll
    for (int i = 0; i < kLook; ++i) fq[i] = fetch(op(i), kb_lds, vp_lds);
    // O is normalised by the sum of exactly the rounded probabilities the
    // P V product uses (a convex combination of V rows even when the
    // dominant probability is not 1 under the lazy reference); the dot
    // products run here, beside the matrix stream, not in the vector block
    float ra[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kPV + kS; ++i) {
      if (i + kLook < kPV + kS) fq[(i + kLook) % (kLook + 1)] = fetch(op(i + kLook), kb_lds, vp_lds);
      product(op(i), fq[i % (kLook + 1)]);
      if (i < kBC / 16) ra[i & 3] = sum_rounded_pairs(pf[i], ra[i & 3]);
    }
    lr_run += (ra[0] + ra[1]) + (ra[2] + ra[3]);
    // order: the first kLook fetches, then (fetch i + kLook, product i); a P V
    // operand takes two LDS reads, a score operand one
    static_assert(kLook % 2 == 0, "slot parity of look-ahead fetches");
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kLook / 2, 0);
#pragma unroll
    for (int i = 0; i < (kPV + kS - kLook) / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kLook; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // first matrix block: S of tile 0 only
  auto mblock_first = [&](const char* kb_lds) {
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
    for (int i = kPV; i < kPV + kS; ++i) product(i, fetch(i, kb_lds, kb_lds));
  };
  // last matrix block: P V of the last tile only (there is no next tile to score)
  auto mblock_last = [&](const char* vp_lds) {
    __builtin_amdgcn_s_setprio(2);
    float ra[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      product(i, fetch(i, vp_lds, vp_lds));
      if (i < kBC / 16) ra[i & 3] = sum_rounded_pairs(pf[i], ra[i & 3]);
    }
    lr_run += (ra[0] + ra[1]) + (ra[2] + ra[3]);
    __builtin_amdgcn_s_setprio(0);
  };

  // vector block: mask, online softmax update, bf16 probabilities of tile j
  auto vblock = [&](int j) {
    if (!live(j)) {
#pragma unroll
      for (int ks = 0; ks < kBC / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)0.0f;
      return;
    }
    const int k0 = (t_lo + j) * kBC;
    const bool need_mask = (k0 + kBC > n_k) || (causal && k0 + kBC - 1 > wq0 + delta) ||
                           (W >= 0 && k0 < wq_last + delta - W);
    if (need_mask) {
      // allowed keys of this lane's row: [lo, hi]; key kj = k0 + 8 half + c
      // is allowed iff 0 <= kj - lo <= hi - lo, one unsigned compare per key
      // (kj < lo wraps to a large value; a row with hi < lo allows none).
      // Compare and select go through VCC one key at a time: left to the
      // compiler, the 32 compares each take a scalar register pair, which
      // this kernel does not have to spare
      int hi = n_k - 1, lo = 0;
      if (causal) hi = min(hi, qi + delta);
      if (W >= 0) lo = max(lo, qi + delta - W);
      const int span = hi - lo;
      const uint32_t e = span < 0 ? 0x80000000u : (uint32_t)(k0 + 8 * half - lo);
      const uint32_t range = span < 0 ? 0u : (uint32_t)span;
      const float ninf = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t t = e + (uint32_t)(kb * 32 + 16 * (r >> 3) + (r & 7));
          float x = sacc[kb][r];
          asm("v_cmp_lt_u32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
              : "+v"(x) : "v"(range), "v"(t), "v"(ninf) : "vcc");
          sacc[kb][r] = x;
        }
    }
    // Probabilities against the current reference max, accepted when this
    // lane's 32 of them sum to at most kLazyBound (so none exceeds it).
    // Otherwise (the row's first live tile, whose reference is -inf, or a
    // jump of the row max) take the tile's true max, rescale the state and
    // recompute.
    float p[kBC / 32][16];
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[kb][r] = exp2_hw(fmaf(sacc[kb][r], c2, -m_run));
    float rsum = tree_sum<kBC / 32>(p);
    if (__builtin_amdgcn_ballot_w64(!(rsum <= kLazyBound)) != 0) {
      const float m_tile = max_halves(tree_max<kBC / 32>(sacc)) * c2;
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_new == m_run ? 1.0f : exp2_hw(m_run - m_new);
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
      const float m_use = m_run == kNegInf ? 0.0f : m_run;
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = exp2_hw(fmaf(sacc[kb][r], c2, -m_use));
      rsum = tree_sum<kBC / 32>(p);
    }
    l_run += rsum;
#pragma unroll
    for (int ks = 0; ks < kBC / 16; ++ks) {
      const int kb = ks >> 1, o8 = (ks & 1) * 8;
      pf[ks] = to_bf16x8(p[kb][o8 + 0], p[kb][o8 + 1], p[kb][o8 + 2], p[kb][o8 + 3],
                         p[kb][o8 + 4], p[kb][o8 + 5], p[kb][o8 + 6], p[kb][o8 + 7]);
    }
  };

  // Step j: tile j has landed in slot j % 4 (each wave waits for its own
  // loads, then the barrier publishes everyone's) and the slot of tile j - 2
  // is free to receive tile j + 2.  Group 0 runs the matrix block of step j
  // and then the vector block of tile j; group 1 the vector block of tile
  // j - 1 and then the matrix block of step j.  The barrier between the two
  // halves keeps the groups half a step apart.
  auto land = [&](int j) {
    if (j + 1 < nt)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * T::kLoads));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    barrier();
  };
  // the slot of tile j - 2 is free once step j has landed; the loads are
  // queued at the end of a vector block, where the wave would otherwise wait
  auto prefetch = [&](int j) {
    if (j + 2 < nt) issue(cur, j + 2, gbase + j + 2);
  };
  // the next item's first tiles and Q fragments: queued once this item's
  // last tile has landed everywhere (its slots gbase + nt, gbase + nt + 1
  // held tiles nt - 4 and nt - 3, which every wave has finished) and the
  // score products no longer read Q
  const bool has_next = !VARLEN && item_id(r_item + 1) < n_items;
  auto next_loads = [&]() {
    if constexpr (!VARLEN) {
      Item nxt;
      if (has_next && make_item(item_id(r_item + 1), nxt)) start_loads(nxt, gbase + nt);
    }
  };

  if (nt > 0) {
    // steps 0 .. nt: step 0 has no previous tile, step nt no next one
    if (group == 0) {
      init_state();
      land(0);
      mblock_first(kslot(gbase));
      barrier();
      vblock(0);
      prefetch(0);
      for (int j = 1; j < nt; ++j) {
        land(j);
        mblock(kslot(gbase + j), vslot(gbase + j - 1));
        barrier();
        vblock(j);
        prefetch(j);
      }
      land(nt);
      next_loads();
      mblock_last(vslot(gbase + nt - 1));
      barrier();  // pairs with group 1's barrier before its last matrix block
    } else {
      land(0);
      if (pend) epilogue(p_og, p_qi, p_nq, p_lse);
      pend = false;
      init_state();
      prefetch(0);
      barrier();
      mblock_first(kslot(gbase));
      for (int j = 1; j < nt; ++j) {
        land(j);
        vblock(j - 1);
        prefetch(j);
        barrier();
        mblock(kslot(gbase + j), vslot(gbase + j - 1));
      }
      land(nt);
      next_loads();
      vblock(nt - 1);
      barrier();
      mblock_last(vslot(gbase + nt - 1));
    }
  } else {
    if (pend) epilogue(p_og, p_qi, p_nq, p_lse);
    pend = false;
    init_state();
    next_loads();
  }

  if (group == 1 && has_next) {
    pend = true;
    p_og = og;
    p_qi = qi;
    p_nq = n_q;
    p_lse = cur.lse_base;
  } else {
    epilogue(og, qi, n_q, cur.lse_base);
  }
  if (!has_next) break;
  gbase += nt;
  ++r_item;
  }
}

template <int D, bool VARLEN, bool KV>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  fwd_bf16_body<D, VARLEN, KV>(a);
}

// The four-wave kernel keeps its reference max while a lane's probabilities
// against it sum to at most this bound: the output u / l does not depend on
// which reference max is used, and probabilities stay <= 2^8.
constexpr float kLazyBound4 = 256.0f;

// Queue the DMA of K/V tile rows [k0, k0 + kBC) of one head straight into
// LDS (no registers).  The buffer descriptor covers only the rows that exist,
// so rows past the sequence end read as zeros without a branch.
template <int D>
__device__ __forceinline__ void issue_tile4(const uint16_t* kg, const uint16_t* vg, long long rs,
                                           int k0, int n_k, char* kdst, char* vdst, int wave,
                                           int lane) {
  using T = BfTile<D, kQThreads>;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const uint32_t nrec =
      __builtin_amdgcn_readfirstlane((uint32_t)min(n_k - k0, kBC) * row_bytes);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(kg + (long long)k0 * rs), 0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(vg + (long long)k0 * rs), 0, nrec, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int blk = i * 4 + wave;  // 1 KB block of the tile written by this wave
    const int slot = blk * 64 + lane;
    const int r = slot / T::kKch;
    const int c = ((slot % T::kKch) ^ tile_swz<D>(r)) & (T::kKch - 1);
    const int cv = ((slot % T::kKch) ^ vtile_swz(r)) & (T::kKch - 1);
    const uint32_t koff = (uint32_t)r * row_bytes + (uint32_t)c * 16;
    const uint32_t voff = (uint32_t)r * row_bytes + (uint32_t)cv * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16, koff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16, voff, 0, 0, 0);
  }
}


template <int D, bool VARLEN, bool KV>
__global__ __launch_bounds__(kQThreads, 2) void fwd_bf16_q_kernel(FwdArgs a) {
  using T = BfTile<D, kQThreads>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps row ranges scalar
  const int half = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;

  Work w;
  if constexpr (VARLEN) {
    if (!varlen_work(a, kQRows, lane, w)) return;
  } else {
    dense_work<KV>(a, ceil_div(a.seqlen_q, kQRows), w, blockIdx.x, gridDim.x);
  }

  const long long rs = (long long)a.heads * D;  // elements between consecutive rows
  const uint16_t* qg = (const uint16_t*)a.q + (w.q_row0 * a.heads + w.h) * D;
  const uint16_t* kg = (const uint16_t*)a.k + (w.k_row0 * a.heads + w.h) * D;
  const uint16_t* vg = (const uint16_t*)a.v + (w.k_row0 * a.heads + w.h) * D;
  uint16_t* og = (uint16_t*)a.o + (w.q_row0 * a.heads + w.h) * D;

  const int n_q = w.n_q, n_k = w.n_k, delta = n_k - n_q;
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2;
  const int q0 = w.qt * kQRows;
  const int q_last = min(q0 + kQRows, n_q) - 1;

  // K/V tiles this query tile needs (fully masked ones are skipped)
  int kv_lo = 0, kv_hi = n_k;
  if (causal) kv_hi = min(kv_hi, q_last + delta + 1);
  if (W >= 0) kv_lo = max(kv_lo, q0 + delta - W);
  const int t_lo = kv_lo / kBC;
  const int t_hi = kv_hi > kv_lo ? ceil_div(kv_hi, kBC) : t_lo;

  // this wave's rows and key range
  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < n_q;
  const int wq_last = min(wq0 + 31, n_q - 1);
  int w_lo = 0, w_hi = n_k;
  if (causal) w_hi = min(w_hi, wq_last + delta + 1);
  if (W >= 0) w_lo = max(w_lo, wq0 + delta - W);
  const int qi = wq0 + l32;  // this lane's query row

  // Q^T operand fragments: lane holds Q[qi][kk*16 + half*8 .. +8]; rows past
  // the sequence read as zeros through the descriptor bound
  bf16x8_t qf[D / 16];
  {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const uint32_t nrec =
        __builtin_amdgcn_readfirstlane((uint32_t)max(min(n_q - wq0, 32), 0) * row_bytes);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(qg + (long long)wq0 * rs), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
          rq, (uint32_t)l32 * row_bytes + (uint32_t)(kk * 16 + half * 8) * 2, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = kNegInf;  // reference max of this row (base-2 scaled)
  float l_run = 0.0f;     // partial exp-sum over this lane-half's keys

  // per-lane parts of the LDS operand addresses
  int k_off[D / 16][kBC / 32];  // K rows enter in pi order (see pi_row)
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb) k_off[kk][kb] = tile_off<D>(kb * 32 + pi_row(l32), kk * 2 + half);
  // V^T fragments through the transposing read: lane j of 16-lane group g
  // addresses row (ks*16 + 8*(g/2) + 4*u + j/4), dims db*32 + 16*(g%2) + 4*(j%4)
  int v_off[D / 32][kBC / 16][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ks = 0; ks < kBC / 16; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = ks * 16 + 8 * (grp >> 1) + 4 * u + (j16 >> 2);
        const int d = db * 32 + 16 * (grp & 1) + 4 * (j16 & 3);
        v_off[db][ks][u] = vtile_off<D>(r, d >> 3) + (d & 7) * 2;
      }

  const int kt_first = max(t_lo, w_lo / kBC);  // the wave's first live tile

  // one K/V tile: S^T = K Q^T, mask, online softmax update, O^T += V^T P^T
  auto compute_tile = [&](int kt, const char* kb_lds, const char* vb_lds) {
    const int k0 = kt * kBC;
    if (!(wave_live && k0 < w_hi && k0 + kBC > w_lo)) return;
    f32x16_t sacc[kBC / 32];
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb) {
        const bf16x8_t kf = *(const bf16x8_t*)(kb_lds + k_off[kk][kb]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
      }
    }

    // element mask, only on tiles crossing a mask boundary.  Key kj = k0 +
    // 8 half + c of this lane's row is allowed iff lo <= kj <= hi, i.e.
    // a_lo <= c <= a_hi with per-lane a_lo = lo - k0 - 8 half and a_hi =
    // hi - k0 - 8 half: one compare of the register's constant offset c with
    // a per-lane value and one select per key, per bound the tile crosses
    const bool cut_hi = (k0 + kBC > n_k) || (causal && k0 + kBC - 1 > wq0 + delta);
    const bool cut_lo = W >= 0 && k0 < wq_last + delta - W;
    if (cut_hi || cut_lo) {
      int hi = n_k - 1, lo = 0;
      if (causal) hi = min(hi, qi + delta);
      if (W >= 0) lo = max(lo, qi + delta - W);
      const int a_hi = hi - k0 - 8 * half, a_lo = lo - k0 - 8 * half;
      if (!cut_lo) {
#pragma unroll
        for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 16 * (r >> 3) + (r & 7) > a_hi) sacc[kb][r] = kNegInf;
      } else if (!cut_hi) {
#pragma unroll
        for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 16 * (r >> 3) + (r & 7) < a_lo) sacc[kb][r] = kNegInf;
      } else {
#pragma unroll
        for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb * 32 + 16 * (r >> 3) + (r & 7);
            if (c > a_hi || c < a_lo) sacc[kb][r] = kNegInf;
          }
      }
    }

    // online softmax update, base 2, lazy reference max: probabilities
    // against the current reference are accepted when this lane's 32 of them
    // sum to at most kLazyBound4 (so none exceeds it); otherwise (a
    // row's first live tile, whose reference is -inf, or a jump of the row
    // max) the reference moves to the tile max, the state is rescaled and
    // the probabilities recomputed
    // the wave's first live tile takes its row max as the reference at once
    // (against -inf every probability would overflow and be recomputed); a
    // row with no allowed key there keeps -inf and goes the slow way below
    if (kt == kt_first) m_run = max_halves(tree_max3<kBC / 32>(sacc)) * c2;
    float p[kBC / 32][16];
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[kb][r] = exp2_hw(fmaf(sacc[kb][r], c2, -m_run));
    float rsum = tree_sum<kBC / 32>(p);
    if (__builtin_amdgcn_ballot_w64(!(rsum <= kLazyBound4)) != 0) {
      const float m_tile = max_halves(tree_max<kBC / 32>(sacc)) * c2;
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_new == m_run ? 1.0f : exp2_hw(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
      const float m_use = m_run == kNegInf ? 0.0f : m_run;
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = exp2_hw(fmaf(sacc[kb][r], c2, -m_use));
      rsum = tree_sum<kBC / 32>(p);
    }
    l_run += rsum;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = p[kb][r];

#pragma unroll
    for (int ks = 0; ks < kBC / 16; ++ks) {
      const int kb = ks >> 1, o8 = (ks & 1) * 8;
      const bf16x8_t pf =
          to_bf16x8(sacc[kb][o8 + 0], sacc[kb][o8 + 1], sacc[kb][o8 + 2], sacc[kb][o8 + 3],
                    sacc[kb][o8 + 4], sacc[kb][o8 + 5], sacc[kb][o8 + 6], sacc[kb][o8 + 7]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(vb_lds + v_off[db][ks][0]));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(vb_lds + v_off[db][ks][1]));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
      }
    }
  };

  if (t_lo < t_hi) {
    issue_tile4<D>(kg, vg, rs, t_lo * kBC, n_k, k_lds0, v_lds0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and tile t_lo are in
    __syncthreads();
    // two tiles per trip so that each buffer is a distinct LDS object
    for (int kt = t_lo; kt < t_hi; kt += 2) {
      if (kt + 1 < t_hi) issue_tile4<D>(kg, vg, rs, (kt + 1) * kBC, n_k, k_lds1, v_lds1, wave, lane);
      compute_tile(kt, k_lds0, v_lds0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (kt + 1 < t_hi) {
        if (kt + 2 < t_hi) issue_tile4<D>(kg, vg, rs, (kt + 2) * kBC, n_k, k_lds0, v_lds0, wave, lane);
        compute_tile(kt + 1, k_lds1, v_lds1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    }
  }

  // epilogue: O = u / l (one division per row), lse = ln 2 * (m + log2 l)
  const float l_tot = sum_halves(l_run);
  if (qi < n_q) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* op = og + (long long)qi * rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        u32x2_t pr;
        pr[0] = pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
        pr[1] = pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
        *(u32x2_t*)(op + d) = pr;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[w.lse_base + qi] = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// fp32 variant: same update, fp32 operands on v_mfma_f32_32x32x2f32 (exact
// fp32 products), probabilities kept in fp32.  4 waves x 32 query rows,
// single-buffered 32-key tiles; dense only.

template <int D>
__global__ __launch_bounds__(kThreads32, 2) void fwd_fp32_kernel(FwdArgs a) {
  constexpr int kStride = D + 1;  // padded LDS row (floats) -> conflict-free column reads
  __shared__ float ks_lds[kBC32 * kStride];
  __shared__ float vs_lds[kBC32 * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  Work w;
  dense_work<false>(a, ceil_div(a.seqlen_q, kBR32), w, blockIdx.x, gridDim.x);
  const long long rs = (long long)a.heads * D;
  const float* qg = (const float*)a.q + (w.q_row0 * a.heads + w.h) * D;
  const float* kg = (const float*)a.k + (w.k_row0 * a.heads + w.h) * D;
  const float* vg = (const float*)a.v + (w.k_row0 * a.heads + w.h) * D;
  float* og = (float*)a.o + (w.q_row0 * a.heads + w.h) * D;

  const int n_q = w.n_q, n_k = w.n_k, delta = n_k - n_q;
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2;
  const int q0 = w.qt * kBR32;
  const int q_last = min(q0 + kBR32, n_q) - 1;
  int kv_lo = 0, kv_hi = n_k;
  if (causal) kv_hi = min(kv_hi, q_last + delta + 1);
  if (W >= 0) kv_lo = max(kv_lo, q0 + delta - W);
  const int t_lo = kv_lo / kBC32;
  const int t_hi = kv_hi > kv_lo ? ceil_div(kv_hi, kBC32) : t_lo;

  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < n_q;
  const int wq_last = min(wq0 + 31, n_q - 1);
  int w_lo = 0, w_hi = n_k;
  if (causal) w_hi = min(w_hi, wq_last + delta + 1);
  if (W >= 0) w_lo = max(w_lo, wq0 + delta - W);
  const int qi = wq0 + l32;

  // Q^T operand: lane holds Q[qi][2*kk + half]
  float qf[D / 2];
  {
    const bool ok = qi < n_q;
    const float* p = qg + (long long)qi * rs + half;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = ok ? p[2 * kk] : 0.0f;
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;

  for (int kt = t_lo; kt < t_hi; ++kt) {
    const int k0 = kt * kBC32;
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < kBC32 * D; e += kThreads32) {
      const int r = e / D, c = e % D;
      const int key = k0 + r;
      const bool ok = key < n_k;
      ks_lds[r * kStride + c] = ok ? kg[(long long)key * rs + c] : 0.0f;
      vs_lds[r * D + c] = ok ? vg[(long long)key * rs + c] : 0.0f;
    }
    __syncthreads();
    if (!(wave_live && k0 < w_hi && k0 + kBC32 > w_lo)) continue;

    // S^T block: register r of lane-half h is key k0 + (r/4)*8 + 4h + r%4
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      const float kf = ks_lds[l32 * kStride + 2 * kk + half];
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[kk], sacc, 0, 0, 0);
    }
    const bool need_mask = (k0 + kBC32 > n_k) || (causal && k0 + kBC32 - 1 > wq0 + delta) ||
                           (W >= 0 && k0 < wq_last + delta - W);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = k0 + (r >> 2) * 8 + 4 * half + (r & 3);
        const bool ok =
            kj < n_k && (!causal || kj <= qi + delta) && (W < 0 || kj >= qi + delta - W);
        if (!ok) sacc[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float rsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_hw(fmaf(sacc[r], c2, -m_use));
      sacc[r] = p;
      rsum += p;
    }
    l_run = fmaf(l_run, alpha, rsum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    // O^T += V^T P^T, two keys per step: register r supplies the pair
    // {(r/4)*8 + r%4, (r/4)*8 + 4 + r%4} through the two lane halves
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = (r >> 2) * 8 + 4 * half + (r & 3);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float vf = vs_lds[key * D + db * 32 + l32];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, sacc[r], oacc[db], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_run + swap_halves(l_run);
  if (qi < n_q) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* op = og + (long long)qi * rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        f32x4_t v4;
        v4[0] = oacc[db][g4 * 4 + 0] * inv;
        v4[1] = oacc[db][g4 * 4 + 1] * inv;
        v4[2] = oacc[db][g4 * 4 + 2] * inv;
        v4[3] = oacc[db][g4 * 4 + 3] * inv;
        *(f32x4_t*)(op + d) = v4;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[w.lse_base + qi] = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : kNegInf;
  }
}

// Compute units of the current device, rounded down to a multiple of 8 (one
// persistent workgroup per CU; 0 if the query fails).
static int persistent_slots() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n & ~7;
}

template <bool VARLEN>
hipError_t launch_bf16_d128(const FwdArgs& a, hipStream_t stream) {
  const int nqt = ceil_div(a.seqlen_q, kBR);
  long long grid = (long long)a.batch * a.heads * nqt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // plain dense launches: one workgroup per CU walks the items (KV-cache
  // launches keep one item per workgroup: their items differ in length in
  // ways a static assignment cannot balance)
  if (!VARLEN && a.seqlens_k == nullptr) {
    const int slots = persistent_slots();
    if (slots >= 8 && grid > slots) grid = slots;
  }
  if (!VARLEN && a.seqlens_k != nullptr)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, false, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<128, VARLEN, false>), dim3((unsigned)grid), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
}

template <bool VARLEN>
hipError_t launch_bf16_d64(const FwdArgs& a, hipStream_t stream) {
  const int nqt = ceil_div(a.seqlen_q, kQRows);
  const long long grid = (long long)a.batch * a.heads * nqt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (!VARLEN && a.seqlens_k != nullptr)
    hipLaunchKernelGGL((fwd_bf16_q_kernel<64, false, true>), dim3((unsigned)grid), dim3(kQThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_q_kernel<64, VARLEN, false>), dim3((unsigned)grid),
                       dim3(kQThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp32_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = ceil_div(a.seqlen_q, kBR32);
  const long long grid = (long long)a.batch * a.heads * nqt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3((unsigned)grid), dim3(kThreads32), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream) {
  const bool varlen = a.cu_q != nullptr;
  if (d == 128) return varlen ? launch_bf16_d128<true>(a, stream) : launch_bf16_d128<false>(a, stream);
  if (d == 64) return varlen ? launch_bf16_d64<true>(a, stream) : launch_bf16_d64<false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_fp32(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_fp32_t<128>(a, stream);
  if (d == 64) return launch_fp32_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
