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
// gfx950 mapping (not from the pages):
//  * 4 waves x 32 query rows per workgroup; each wave owns whole rows, so row
//    statistics need no LDS traffic (one lane-half swap per tile for the max).
//  * Scores are produced transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    each lane then holds 16 keys of a single query row, so the row max/sum is
//    mostly in-lane, and the output accumulator O^T = V^T P^T gives each lane
//    a single query row as well (one rescale factor per lane).
//  * K rows enter the score product in a permuted order so that a lane's
//    probabilities are already the k-slots the P V product wants: no data
//    movement between the two products.
//  * The softmax works in base 2 with log2(e) folded into the scale
//    (v_exp_f32), moves its reference max only when a row max grows by more
//    than 2^8, and divides once per row at the end.
//  * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//    destination, no register staging; rows past the sequence end come back
//    as zeros from the descriptor bound), double buffered, one barrier per
//    tile.  V stays row-major in LDS: the P V operand is read with the
//    transposing LDS read (ds_read_b64_tr_b16).  K and V use different
//    16-byte-chunk swizzles, each chosen so that its own read pattern is free
//    of LDS bank conflicts.
//  * Fully masked K/V tiles (causal, sliding window) are never loaded;
//    element masks run only on tiles that cross a mask boundary.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per K/V tile
constexpr int kThreads = 256;

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

__device__ __forceinline__ void dense_work(const FwdArgs& a, int nqt, Work& w) {
  const int id = xcd_contiguous(blockIdx.x, gridDim.x);
  const int bh = id / nqt;
  const int t = id - bh * nqt;
  const int b = bh / a.heads;
  w.h = bh - b * a.heads;
  w.qt = nqt - 1 - t;  // longest (causal) tiles first
  w.n_q = a.seqlen_q;
  w.n_k = a.seqlen_k;
  w.q_row0 = (long long)b * a.seqlen_q;
  w.k_row0 = (long long)b * a.seqlen_k;
  w.lse_base = ((long long)b * a.heads + w.h) * a.seqlen_q;
}

// Variable-length scheduler: every wave scans the per-sequence tile counts
// ceil(len_q / kBR) from cu_seqlens_q (no host round trip), drops the
// workgroups past the live total, renumbers the rest XCD-contiguously and
// finds its (head, sequence, tile).  Head-major order keeps the tiles of one
// (sequence, head) on one XCD.
__device__ bool varlen_work(const FwdArgs& a, int lane, Work& w) {
  const int nseq = a.batch;
  int total = 0;
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    const int s = s0 + lane;
    const int nt = s < nseq ? ceil_div(max(a.cu_q[s + 1] - a.cu_q[s], 0), kBR) : 0;
    const int inc = wave_inclusive_scan(nt, lane);
    total += __shfl(inc, 63, 64);
  }
  const long long live = (long long)total * a.heads;
  if ((long long)blockIdx.x >= live) return false;
  const int id = xcd_contiguous(blockIdx.x, (int)live);
  w.h = id / total;
  const int g = id - w.h * total;
  int base = 0;
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    const int s = s0 + lane;
    const int nt = s < nseq ? ceil_div(max(a.cu_q[s + 1] - a.cu_q[s], 0), kBR) : 0;
    const int inc = wave_inclusive_scan(nt, lane) + base;
    const int exc = inc - nt;
    const unsigned long long hit = __ballot(s < nseq && g >= exc && g < inc);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int seq = s0 + src;
      const int t = g - __shfl(exc, src, 64);
      const int ntq = __shfl(nt, src, 64);
      const int cq0 = a.cu_q[seq], cq1 = a.cu_q[seq + 1];
      const int ck0 = a.cu_k[seq], ck1 = a.cu_k[seq + 1];
      w.qt = ntq - 1 - t;
      w.n_q = cq1 - cq0;
      w.n_k = max(ck1 - ck0, 0);
      w.q_row0 = cq0;
      w.k_row0 = ck0;
      w.lse_base = (long long)w.h * a.cu_q[nseq] + cq0;
      return true;
    }
    base = __shfl(inc, 63, 64);
  }
  return false;
}

// One K or V tile in LDS: kBC rows x D bf16, row-major as in HBM; 16-byte
// chunk c of row r sits at chunk position c ^ tile_swz(r) so that the MFMA
// operand reads of a wave spread over the LDS banks.
template <int D>
struct BfTile {
  static constexpr int kKch = D / 8;                    // 16-byte chunks per row
  static constexpr int kBytes = kBC * D * 2;            // one tile
  static constexpr int kLoads = kBytes / 16 / kThreads; // 16-byte DMA loads per thread per tile
  static_assert(kBytes % (16 * kThreads) == 0, "tile must split evenly over the threads");
};

__device__ __forceinline__ int tile_swz(int r) {
  return (r & 3) | ((r >> 1) & 4) | ((r << 1) & 8);
}

template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + ((c ^ tile_swz(r)) & (D / 8 - 1)) * 16;
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

// Queue the DMA of K/V tile rows [k0, k0 + kBC) of one head straight into
// LDS (no registers).  The buffer descriptor covers only the rows that exist,
// so rows past the sequence end read as zeros without a branch.
template <int D>
__device__ __forceinline__ void issue_tile(const uint16_t* kg, const uint16_t* vg, long long rs,
                                           int k0, int n_k, char* kdst, char* vdst, int wave,
                                           int lane) {
  using T = BfTile<D>;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const uint32_t nrec = (uint32_t)min(n_k - k0, kBC) * row_bytes;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kg + (long long)k0 * rs), 0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vg + (long long)k0 * rs), 0, nrec, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) {
    const int blk = i * 4 + wave;  // 1 KB block of the tile written by this wave
    const int slot = blk * 64 + lane;
    const int r = slot / T::kKch;
    const int c = ((slot % T::kKch) ^ tile_swz(r)) & (T::kKch - 1);
    const int cv = ((slot % T::kKch) ^ vtile_swz(r)) & (T::kKch - 1);
    const uint32_t koff = (uint32_t)r * row_bytes + (uint32_t)c * 16;
    const uint32_t voff = (uint32_t)r * row_bytes + (uint32_t)cv * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16, koff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16, voff, 0, 0, 0);
  }
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

// The running max is moved only when a row's new max exceeds it by more than
// this (base-2 units): the output u / l does not depend on which reference
// max is used, and probabilities stay <= 2^8, far from fp32/bf16 overflow.
constexpr float kRescaleSlack = 8.0f;

template <int D, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using T = BfTile<D>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;

  Work w;
  if constexpr (VARLEN) {
    if (!varlen_work(a, lane, w)) return;
  } else {
    dense_work(a, ceil_div(a.seqlen_q, kBR), w);
  }

  const long long rs = (long long)a.heads * D;  // elements between consecutive rows
  const uint16_t* qg = (const uint16_t*)a.q + (w.q_row0 * a.heads + w.h) * D;
  const uint16_t* kg = (const uint16_t*)a.k + (w.k_row0 * a.heads + w.h) * D;
  const uint16_t* vg = (const uint16_t*)a.v + (w.k_row0 * a.heads + w.h) * D;
  uint16_t* og = (uint16_t*)a.o + (w.q_row0 * a.heads + w.h) * D;

  const int n_q = w.n_q, n_k = w.n_k, delta = n_k - n_q;
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2;
  const int q0 = w.qt * kBR;
  const int q_last = min(q0 + kBR, n_q) - 1;

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
    const uint32_t nrec = (uint32_t)max(min(n_q - wq0, 32), 0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qg + (long long)wq0 * rs), 0, nrec, kRsrcWord3);
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

    // element mask, only on tiles crossing a mask boundary
    const bool need_mask = (k0 + kBC > n_k) || (causal && k0 + kBC - 1 > wq0 + delta) ||
                           (W >= 0 && k0 < wq_last + delta - W);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + kb * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
          const bool ok = kj < n_k && (!causal || kj <= qi + delta) &&
                          (W < 0 || kj >= qi + delta - W);
          if (!ok) sacc[kb][r] = kNegInf;
        }
    }

    // online softmax update, base 2, lazy reference max
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    const float m_tile = max_halves(mx) * c2;
    const bool grow = m_tile > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? m_tile : m_run;
      const float alpha = grow ? exp2_hw(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.0f : m_run;
    float rsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(fmaf(sacc[kb][r], c2, -m_use));
        sacc[kb][r] = p;
        rsum += p;
      }
    l_run += rsum;

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
    issue_tile<D>(kg, vg, rs, t_lo * kBC, n_k, k_lds0, v_lds0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and tile t_lo are in
    __syncthreads();
    // two tiles per trip so that each buffer is a distinct LDS object
    for (int kt = t_lo; kt < t_hi; kt += 2) {
      if (kt + 1 < t_hi) issue_tile<D>(kg, vg, rs, (kt + 1) * kBC, n_k, k_lds1, v_lds1, wave, lane);
      compute_tile(kt, k_lds0, v_lds0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (kt + 1 < t_hi) {
        if (kt + 2 < t_hi) issue_tile<D>(kg, vg, rs, (kt + 2) * kBC, n_k, k_lds0, v_lds0, wave, lane);
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
// fp32 variant: same tiling and update, fp32 operands on
// v_mfma_f32_32x32x2f32 (exact fp32 products), probabilities kept in fp32.
// Single-buffered 32-key tiles; dense only.

constexpr int kBC32 = 32;

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp32_kernel(FwdArgs a) {
  constexpr int kStride = D + 1;  // padded LDS row (floats) -> conflict-free column reads
  __shared__ float ks_lds[kBC32 * kStride];
  __shared__ float vs_lds[kBC32 * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  Work w;
  dense_work(a, ceil_div(a.seqlen_q, kBR), w);
  const long long rs = (long long)a.heads * D;
  const float* qg = (const float*)a.q + (w.q_row0 * a.heads + w.h) * D;
  const float* kg = (const float*)a.k + (w.k_row0 * a.heads + w.h) * D;
  const float* vg = (const float*)a.v + (w.k_row0 * a.heads + w.h) * D;
  float* og = (float*)a.o + (w.q_row0 * a.heads + w.h) * D;

  const int n_q = w.n_q, n_k = w.n_k, delta = n_k - n_q;
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2;
  const int q0 = w.qt * kBR;
  const int q_last = min(q0 + kBR, n_q) - 1;
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
    for (int e = tid; e < kBC32 * D; e += kThreads) {
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

template <int D, bool VARLEN>
hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = ceil_div(a.seqlen_q, kBR);
  const long long grid = (long long)a.batch * a.heads * nqt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, VARLEN>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp32_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = ceil_div(a.seqlen_q, kBR);
  const long long grid = (long long)a.batch * a.heads * nqt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream) {
  const bool varlen = a.cu_q != nullptr;
  if (d == 128) return varlen ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
  if (d == 64) return varlen ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_fp32(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_fp32_t<128>(a, stream);
  if (d == 64) return launch_fp32_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
