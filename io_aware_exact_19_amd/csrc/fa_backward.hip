// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale Q K^T) V for
// an output gradient dO, recomputing the probabilities from the row
// log-sum-exp the forward pass emits instead of storing them -- the reason
// the forward keeps lse ("FlashAttention" (aiwiki.page), section "Training
// and computational complexity").  With P = exp(scale Q K^T - lse) (zero on
// masked pairs) the gradients are the chain rule through the softmax:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id (= rowsum(P o dP)),
//   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, no atomics (every output element has one writer):
//  * prep: D_i and the base-2 lse (lse * log2 e) per row, into the workspace.
//  * dkdv: one workgroup of 4 waves per (batch, head, 128 keys); each wave
//    owns 32 keys and keeps their K and V fragments in registers while
//    64-row tiles of Q and dO stream through LDS.  Per 32 query rows it
//    forms S = Q K^T and dP = dO V^T (keys in the lane, rows in the
//    accumulator registers), P and dS on the VALU, then accumulates
//    dV^T += dO^T P and dK^T += Q^T dS with the tile read transposed.
//  * dq: one workgroup per (batch, head, 128 query rows); each wave owns 32
//    rows (Q and dO fragments in registers) while 64-key tiles of K and V
//    stream through LDS: S^T = K Q^T, dP^T = V dO^T, dS^T on the VALU, then
//    dQ^T += K^T dS^T.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 before they enter a product.  The operand layouts are
// those of the forward kernel: the query (or key) rows that form a score
// accumulator enter in pi order (bits 2 and 3 of the row index swapped), so
// each lane's accumulator registers are directly the k-slots of the next
// product's operand, and transposed operands come from ds_read_b64_tr_b16.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) float lds_float_t;

constexpr int kBThreads = 256;  // 4 waves
constexpr int kWaveRows = 32;   // keys (dkdv) or query rows (dq) owned by one wave
constexpr int kTile = 64;       // rows of a streamed LDS tile
constexpr int kRsrcWord3 = 0x00020000;

// The 32 rows behind a 32x32 score accumulator enter in this order, so that
// lane half h, register r holds logical row 16 (r / 8) + 8 h + (r % 8).
__device__ __forceinline__ int pi_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// LDS tile of kTile rows x D bf16, rows padded by 16 bytes
template <int D>
constexpr int row_stride() { return D * 2 + 16; }

// buffer descriptor over [p, p + bytes); offsets past the end read zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// rows [row0, row0 + kTile) of a [rows][heads][D] bf16 tensor (head base g,
// rs elements between rows) into an LDS tile; rows >= n become zeros
template <int D>
__device__ __forceinline__ void stage_tile(char* lds, const uint16_t* g, long long rs, int row0,
                                           int n, int tid) {
  constexpr int kCh = D / 8;                    // 16-byte chunks per row
  constexpr int kPer = kTile * kCh / kBThreads;  // chunks per thread
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const int rows = max(min(n - row0, kTile), 0);
  const __amdgpu_buffer_rsrc_t r = rsrc_of(g + (long long)max(row0, 0) * rs, (uint32_t)rows * row_bytes);
  u32x4_t x[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * kBThreads + tid, row = c / kCh, ch = c % kCh;
    x[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)row * row_bytes + ch * 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * kBThreads + tid, row = c / kCh, ch = c % kCh;
    *(lds_bf16x8_t*)((lds_void_t*)(lds + row * row_stride<D>() + ch * 16)) =
        __builtin_bit_cast(bf16x8_t, x[i]);
  }
}

// Operand fragment with rows as the reduction index, read transposed from an
// LDS tile: lane l gets tile[row0 + 8 h + 0..7][32 db + l % 32] for the
// k-slice starting at row0 (h = lane half); row0 is a multiple of 16.
template <int D>
__device__ __forceinline__ bf16x8_t tr_frag(const char* lds, int row0, int db, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = row0 + 8 * (g >> 1) + (j >> 2);
  const int d = db * 32 + 16 * (g & 1) + 4 * (j & 3);
  const char* p = lds + row * row_stride<D>() + d * 2;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_void_t*)p));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_t*)((lds_void_t*)(p + 4 * row_stride<D>())));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Operand fragment with d as the reduction index: tile[row][16 kk + 8 h .. + 7]
template <int D>
__device__ __forceinline__ bf16x8_t row_frag(const char* lds, int row, int kk, int half) {
  return *(const lds_bf16x8_t*)((const lds_void_t*)(lds + row * row_stride<D>() + (kk * 16 + half * 8) * 2));
}

// key j allowed for query i (delta = n_k - n_q)
__device__ __forceinline__ bool allowed(const BwdArgs& a, int i, int j, int delta) {
  return i < a.seqlen_q && j < a.seqlen_k && (!a.causal || j <= i + delta) &&
         (a.window_left < 0 || j >= i + delta - a.window_left);
}

// ---------------------------------------------------------------- prep
template <int D>
__global__ __launch_bounds__(kBThreads) void bwd_prep_kernel(BwdArgs a) {
  const long long idx = (long long)blockIdx.x * kBThreads + threadIdx.x;  // (b, h, i) of [B, H, n_q]
  const long long total = (long long)a.batch * a.heads * a.seqlen_q;
  if (idx >= total) return;
  const int i = (int)(idx % a.seqlen_q);
  const long long bh = idx / a.seqlen_q;
  const int h = (int)(bh % a.heads), b = (int)(bh / a.heads);
  const long long off = (((long long)b * a.seqlen_q + i) * a.heads + h) * D;
  const u32x4_t* op = (const u32x4_t*)((const uint16_t*)a.o + off);
  const u32x4_t* gp = (const u32x4_t*)((const uint16_t*)a.dout + off);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4_t x = op[c], y = gp[c];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s = fmaf(bf16_lo(x[j]), bf16_lo(y[j]), fmaf(bf16_hi(x[j]), bf16_hi(y[j]), s));
  }
  a.ws_d[idx] = s;
  a.ws_l2[idx] = a.lse[idx] * kLog2e;  // -inf (a row with no key) stays -inf
}

// ---------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kRS = row_stride<D>();
  __shared__ __attribute__((aligned(16))) char q_lds[kTile * kRS];
  __shared__ __attribute__((aligned(16))) char g_lds[kTile * kRS];  // dO tile
  __shared__ __attribute__((aligned(16))) float l2_lds[kTile];
  __shared__ __attribute__((aligned(16))) float d_lds[kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = a.heads, n_q = a.seqlen_q, n_k = a.seqlen_k, delta = n_k - n_q;
  const int nkt = ceil_div(n_k, 4 * kWaveRows);
  const int kt = blockIdx.x % nkt;
  const int bh = blockIdx.x / nkt;
  const int h = bh % H, b = bh / H;
  const long long rs = (long long)H * D;
  const int k0 = kt * 4 * kWaveRows;
  const int wk0 = k0 + wave * kWaveRows;
  const int key = wk0 + l32;  // this lane's key

  // K^T and V^T operand fragments of this lane's key (rows past n_k are zero)
  const uint16_t* kg = (const uint16_t*)a.k + ((long long)b * n_k * H + h) * D;
  const uint16_t* vg = (const uint16_t*)a.v + ((long long)b * n_k * H + h) * D;
  bf16x8_t kf[D / 16], vf[D / 16];
  {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const uint32_t nrec = (uint32_t)max(min(n_k - wk0, kWaveRows), 0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rk = rsrc_of(kg + (long long)max(wk0, 0) * rs, nrec);
    const __amdgpu_buffer_rsrc_t rv = rsrc_of(vg + (long long)max(wk0, 0) * rs, nrec);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint32_t off = (uint32_t)l32 * row_bytes + (uint32_t)(kk * 16 + half * 8) * 2;
      kf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  }

  f32x16_t dkacc[D / 32], dvacc[D / 32];  // dK^T, dV^T: [d][key], lane = key
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.0f;
      dvacc[db][r] = 0.0f;
    }

  // query rows that can see one of the workgroup's keys
  int q_lo = 0, q_hi = n_q;
  if (a.causal) q_lo = max(q_lo, k0 - delta);
  if (a.window_left >= 0) q_hi = min(q_hi, k0 + 4 * kWaveRows - delta + a.window_left);
  const uint16_t* qg = (const uint16_t*)a.q + ((long long)b * n_q * H + h) * D;
  const uint16_t* gg = (const uint16_t*)a.dout + ((long long)b * n_q * H + h) * D;
  const float* l2g = a.ws_l2 + ((long long)b * H + h) * n_q;
  const float* dg = a.ws_d + ((long long)b * H + h) * n_q;
  const float c2 = a.scale_log2;

  for (int q0 = (max(q_lo, 0) / kTile) * kTile; q0 < q_hi; q0 += kTile) {
    stage_tile<D>(q_lds, qg, rs, q0, n_q, tid);
    stage_tile<D>(g_lds, gg, rs, q0, n_q, tid);
    if (tid < kTile) {
      const int i = q0 + tid;
      // rows past n_q: +inf makes P = 0 (they are masked anyway)
      ((lds_float_t*)(lds_void_t*)l2_lds)[tid] = i < n_q ? l2g[i] : __builtin_inff();
      ((lds_float_t*)(lds_void_t*)d_lds)[tid] = i < n_q ? dg[i] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kTile / 32; ++rb) {
      f32x16_t sacc = {}, dpacc = {};
      const int prow = rb * 32 + pi_row(l32);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(q_lds, prow, kk, half), kf[kk], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(g_lds, prow, kk, half), vf[kk], dpacc, 0, 0, 0);
      }
      // register r of lane half h holds tile row rb*32 + 16 (r/8) + 8 h + r%8
      bf16x8_t pf[2], sf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int t0 = rb * 32 + 16 * ks + 8 * half;
        float p[8], ds[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float l2 = ((const lds_float_t*)(const lds_void_t*)l2_lds)[t0 + t];
          const float dd = ((const lds_float_t*)(const lds_void_t*)d_lds)[t0 + t];
          const int r = 8 * ks + t;
          const bool ok = allowed(a, q0 + t0 + t, key, delta);
          p[t] = ok ? exp2_hw(fmaf(sacc[r], c2, -l2)) : 0.0f;
          ds[t] = p[t] * (dpacc[r] - dd);
        }
        pf[ks] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        sf[ks] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
      // dV^T += dO^T P, dK^T += Q^T dS over these 32 rows
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(g_lds, rb * 32 + 16 * ks, db, lane), pf[ks], dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(q_lds, rb * 32 + 16 * ks, db, lane), sf[ks], dkacc[db], 0, 0, 0);
        }
    }
    __syncthreads();
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
        pk[0] = pack_bf16x2(a.scale * dkacc[db][g4 * 4 + 0], a.scale * dkacc[db][g4 * 4 + 1]);
        pk[1] = pack_bf16x2(a.scale * dkacc[db][g4 * 4 + 2], a.scale * dkacc[db][g4 * 4 + 3]);
        pv[0] = pack_bf16x2(dvacc[db][g4 * 4 + 0], dvacc[db][g4 * 4 + 1]);
        pv[1] = pack_bf16x2(dvacc[db][g4 * 4 + 2], dvacc[db][g4 * 4 + 3]);
        *(u32x2_t*)(dkp + d) = pk;
        *(u32x2_t*)(dvp + d) = pv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int kRS = row_stride<D>();
  __shared__ __attribute__((aligned(16))) char k_lds[kTile * kRS];
  __shared__ __attribute__((aligned(16))) char v_lds[kTile * kRS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = a.heads, n_q = a.seqlen_q, n_k = a.seqlen_k, delta = n_k - n_q;
  const int nqt = ceil_div(n_q, 4 * kWaveRows);
  const int qt = blockIdx.x % nqt;
  const int bh = blockIdx.x / nqt;
  const int h = bh % H, b = bh / H;
  const long long rs = (long long)H * D;
  const int q0 = qt * 4 * kWaveRows;
  const int wq0 = q0 + wave * kWaveRows;
  const int row = wq0 + l32;  // this lane's query row

  // Q^T and dO^T operand fragments of this lane's row (rows past n_q are zero)
  const uint16_t* qg = (const uint16_t*)a.q + ((long long)b * n_q * H + h) * D;
  const uint16_t* gg = (const uint16_t*)a.dout + ((long long)b * n_q * H + h) * D;
  bf16x8_t qf[D / 16], gf[D / 16];
  {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const uint32_t nrec = (uint32_t)max(min(n_q - wq0, kWaveRows), 0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rq = rsrc_of(qg + (long long)max(wq0, 0) * rs, nrec);
    const __amdgpu_buffer_rsrc_t rg = rsrc_of(gg + (long long)max(wq0, 0) * rs, nrec);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint32_t off = (uint32_t)l32 * row_bytes + (uint32_t)(kk * 16 + half * 8) * 2;
      qf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      gf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
    }
  }
  const bool row_live = row < n_q;
  const float l2 = row_live ? a.ws_l2[((long long)b * H + h) * n_q + row] : __builtin_inff();
  const float dd = row_live ? a.ws_d[((long long)b * H + h) * n_q + row] : 0.0f;

  f32x16_t dqacc[D / 32];  // dQ^T: [d][row], lane = row
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.0f;

  // keys the workgroup's rows can see
  const int q_last = min(q0 + 4 * kWaveRows, n_q) - 1;
  int k_lo = 0, k_hi = n_k;
  if (a.causal) k_hi = min(k_hi, q_last + delta + 1);
  if (a.window_left >= 0) k_lo = max(k_lo, q0 + delta - a.window_left);
  const uint16_t* kg = (const uint16_t*)a.k + ((long long)b * n_k * H + h) * D;
  const uint16_t* vg = (const uint16_t*)a.v + ((long long)b * n_k * H + h) * D;
  const float c2 = a.scale_log2;

  for (int k0 = (max(k_lo, 0) / kTile) * kTile; k0 < k_hi; k0 += kTile) {
    stage_tile<D>(k_lds, kg, rs, k0, n_k, tid);
    stage_tile<D>(v_lds, vg, rs, k0, n_k, tid);
    __syncthreads();
    f32x16_t sacc[kTile / 32], dpacc[kTile / 32];
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      sacc[kb] = f32x16_t{};
      dpacc[kb] = f32x16_t{};
      const int prow = kb * 32 + pi_row(l32);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(k_lds, prow, kk, half), qf[kk], sacc[kb], 0, 0, 0);
        dpacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(v_lds, prow, kk, half), gf[kk], dpacc[kb], 0, 0, 0);
      }
    }
    // register r of lane half h holds key k0 + 32 kb + 16 (r/8) + 8 h + r%8
    bf16x8_t sf[kTile / 16];
#pragma unroll
    for (int ks = 0; ks < kTile / 16; ++ks) {
      const int kb = ks >> 1, o8 = (ks & 1) * 8;
      float ds[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = o8 + t;
        const int key = k0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
        const bool ok = allowed(a, row, key, delta);
        const float p = ok ? exp2_hw(fmaf(sacc[kb][r], c2, -l2)) : 0.0f;
        ds[t] = p * (dpacc[kb][r] - dd);
      }
      sf[ks] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    }
    // dQ^T += K^T dS^T over these keys
#pragma unroll
    for (int ks = 0; ks < kTile / 16; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(k_lds, 16 * ks, db, lane), sf[ks], dqacc[db], 0, 0, 0);
    __syncthreads();
  }

  if (row_live) {
    uint16_t* qp = (uint16_t*)a.dq + (((long long)b * n_q + row) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        u32x2_t pq;
        pq[0] = pack_bf16x2(a.scale * dqacc[db][g4 * 4 + 0], a.scale * dqacc[db][g4 * 4 + 1]);
        pq[1] = pack_bf16x2(a.scale * dqacc[db][g4 * 4 + 2], a.scale * dqacc[db][g4 * 4 + 3]);
        *(u32x2_t*)(qp + d) = pq;
      }
  }
}

template <int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.batch * a.heads * a.seqlen_q;
  const long long g0 = (rows + kBThreads - 1) / kBThreads;
  const long long g1 = (long long)a.batch * a.heads * ceil_div(a.seqlen_k, 4 * kWaveRows);
  const long long g2 = (long long)a.batch * a.heads * ceil_div(a.seqlen_q, 4 * kWaveRows);
  if (g0 > 0x7fffffffLL || g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g0 > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)g0), dim3(kBThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g1 > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)g1), dim3(kBThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g2 > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)g2), dim3(kBThreads), 0, stream, a);
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
