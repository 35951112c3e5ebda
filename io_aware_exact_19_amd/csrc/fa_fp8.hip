// FP8 attention forward (prefill) for gfx950: Q, K, V in OCP e4m3 with one
// dequantisation factor per (batch, head) and tensor, output bf16.
//
// Same tiled evaluation with online normalisation as the bf16 kernels
// ("FlashAttention" (aiwiki.page), section "Tiling and online normalisation";
// the low-precision variant is the FP8 path named in its section "Versions"),
// with both matrix products on v_mfma_scale_f32_32x32x64_f8f6f4 (fp32
// accumulation, unit block scales):
//   S = (scale * dq * dk) * Q8 K8^T, P = softmax(S) (fp32, base 2, lazy
//   reference max), P rounded to e4m3, O = dv * (P8 V8) / sum(P8).
//
// gfx950 mapping (not from the pages):
//  * The two operands of the fp8 matrix instruction share one (lane half,
//    byte) -> k map, and its 32x32 accumulator gives lane (h, n) the rows
//    8 (r / 4) + 4 h + r % 4.  Loading the K rows of each 32-key block in the
//    order key(kb, i) = 32 ((i >> 2) & 1) + 16 kb + 4 (i >> 3) + (i & 3)
//    makes the 32 probabilities of lane (h, n) the keys 32 h + [0, 32) of the
//    64-key tile, in register order, which is exactly the k operand layout of
//    the P V product: no data movement between the two products.
//  * The P V operand then wants 32 consecutive keys of one head dimension:
//    the V tile stays row-major in LDS and four 8-bit transposing reads
//    (ds_read_b64_tr_b8: in each 16-lane group lane j addresses row j / 2,
//    bytes 8 (j % 2), and receives byte column j of the 8 x 16 block, rows in
//    order) gather 8 keys each.
//  * The row sums of the rounded probabilities come from one more matrix
//    product per tile (an operand of e4m3 ones), not from vector work.
//  * The first product of each score chain takes a zero block held in
//    registers as its accumulator input, and its K operand is kept live
//    until after the product: when the result registers are not tied to the
//    accumulator input this compiler lets them overlap the operand registers
//    of the same instruction, which reads back garbage.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kD8 = 128;            // head dimension
constexpr int kBC8 = 64;            // keys per tile
constexpr int kWaves8 = 4;
constexpr int kThreads8 = kWaves8 * 64;
constexpr int kRows8 = kWaves8 * 32;  // query rows per workgroup
constexpr int kTile8 = kBC8 * kD8;    // bytes of one K or V tile (8 KB)
constexpr int kLoads8 = kTile8 / 16 / kThreads8;  // 16-byte loads per thread per tile
constexpr int kRsrcWord3 = 0x00020000;            // raw buffer, 32-bit data format
constexpr float kLazyBound8 = 256.0f;  // probabilities stay <= 2^8, inside e4m3's 448
constexpr int kScaleOne = 127;         // E8M0 block scale 2^0

__device__ __forceinline__ f32x16_t mma8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, kScaleOne);
}

// LDS position of 16-byte chunk c of K tile row r (8 chunks per 128-byte row):
// the 16 rows one 16-lane group reads land in distinct bank groups
__device__ __forceinline__ int k8_swz(int r) { return ((r >> 1) & 3) | ((r >> 3) & 4); }
// V tile row r (key): a 32-lane transposing read covers 8 rows x 2 adjacent
// chunks (2 db, 2 db + 1), two rows per 256-byte bank line; XOR with an even
// value keeps each row's pair a pair, so the 4 rows of each parity land on 4
// disjoint pairs of bank groups (XOR with 1 would map a pair onto itself)
__device__ __forceinline__ int v8_swz(int r) { return ((r >> 1) & 3) << 1; }

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

struct Fp8Args {
  const uint8_t* q;     // [batch, seqlen_q, heads, 128] e4m3
  const uint8_t* k;     // [batch, seqlen_k, heads, 128] e4m3
  const uint8_t* v;     // [batch, seqlen_k, heads, 128] e4m3
  uint16_t* o;          // [batch, seqlen_q, heads, 128] bf16
  float* lse;           // [batch, heads, seqlen_q] or null
  const float* dq;      // [batch * heads] dequantisation factors
  const float* dk;
  const float* dv;
  int batch, heads, seqlen_q, seqlen_k;
  float scale_log2;     // scale * log2(e)
  int causal, window_left;
};

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__global__ __launch_bounds__(kThreads8, 2) void fwd_fp8_kernel(Fp8Args a) {
  __shared__ __attribute__((aligned(1024))) char k_lds0[kTile8];
  __shared__ __attribute__((aligned(1024))) char k_lds1[kTile8];
  __shared__ __attribute__((aligned(1024))) char v_lds0[kTile8];
  __shared__ __attribute__((aligned(1024))) char v_lds1[kTile8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // work item: (batch, head, query tile).  Workgroup i reaches XCD i % 8,
  // which starts its workgroups in order as CUs free up; every head keeps its
  // tiles on one XCD (shared L2).  With a mask the tiles differ in length:
  // XCD x takes the heads x, x + 8, ... and starts all their tiles longest
  // first (longest-processing-time order); otherwise the ids are numbered
  // XCD-contiguously.
  const int nqt = ceil_div(a.seqlen_q, kRows8);
  const int nbh = a.batch * a.heads;
  int bh, t;  // t: rank of the tile in start order
  if ((a.causal || a.window_left >= 0) && nbh % 8 == 0) {
    const int x = blockIdx.x & 7, kx = blockIdx.x >> 3, hx = nbh >> 3;
    t = kx / hx;
    bh = x + 8 * (kx - t * hx);
  } else {
    const int id = xcd_contiguous(blockIdx.x, gridDim.x);
    bh = id / nqt;
    t = id - bh * nqt;
  }
  const int b = bh / a.heads, h = bh - b * a.heads;
  // causal: later tiles see more keys; a left window without the causal
  // bound: earlier tiles see more keys
  const int qt = a.causal || a.window_left < 0 ? nqt - 1 - t : t;
  const int n_q = a.seqlen_q, n_k = a.seqlen_k, delta = n_k - n_q;
  const int causal = a.causal, W = a.window_left;
  const float c2 = a.scale_log2 * a.dq[bh] * a.dk[bh];
  const float vscale = a.dv[bh];
  const uint32_t row_bytes = (uint32_t)(a.heads * kD8);
  const uint8_t* qg = a.q + ((long long)b * n_q * a.heads + h) * kD8;
  const uint8_t* kg = a.k + ((long long)b * n_k * a.heads + h) * kD8;
  const uint8_t* vg = a.v + ((long long)b * n_k * a.heads + h) * kD8;
  uint16_t* og = a.o + ((long long)b * n_q * a.heads + h) * kD8;

  const int q0 = qt * kRows8;
  const int q_last = min(q0 + kRows8, n_q) - 1;
  int kv_lo = 0, kv_hi = n_k;
  if (causal) kv_hi = min(kv_hi, q_last + delta + 1);
  if (W >= 0) kv_lo = max(kv_lo, q0 + delta - W);
  const int t_lo = kv_lo / kBC8;
  const int t_hi = kv_hi > kv_lo ? ceil_div(kv_hi, kBC8) : t_lo;

  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < n_q;
  const int wq_last = min(wq0 + 31, n_q - 1);
  int w_lo = 0, w_hi = n_k;
  if (causal) w_hi = min(w_hi, wq_last + delta + 1);
  if (W >= 0) w_lo = max(w_lo, wq0 + delta - W);
  const int qi = wq0 + l32;

  // Q^T operand: lane (h, n) holds bytes 64 kk + 32 h + [0, 32) of row qi
  i32x8_t qf[2];
  {
    const uint32_t nrec =
        __builtin_amdgcn_readfirstlane((uint32_t)max(min(n_q - wq0, 32), 0) * row_bytes);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qg + (long long)wq0 * row_bytes), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (uint32_t)l32 * row_bytes + (uint32_t)(64 * kk + 32 * half + 16 * p), 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) qf[kk][4 * p + w] = (int)x[w];
      }
  }

  // tile loads straight into LDS (16 bytes per lane, swizzled chunk order)
  auto issue = [&](int kt, char* kdst, char* vdst) {
    const int k0 = kt * kBC8;
    const uint32_t nrec = (uint32_t)min(n_k - k0, kBC8) * row_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kg + (long long)k0 * row_bytes), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vg + (long long)k0 * row_bytes), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kLoads8; ++i) {
      const int blk = i * kWaves8 + wave;
      const int s = blk * 64 + lane;
      const int r = s >> 3;
      const int ck = (s & 7) ^ k8_swz(r), cv = ((s & 7) ^ v8_swz(r)) & 7;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16,
                                               (uint32_t)r * row_bytes + (uint32_t)ck * 16, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16,
                                               (uint32_t)r * row_bytes + (uint32_t)cv * 16, 0, 0, 0);
    }
  };

  // per-lane LDS offsets of the operand fragments
  int k_off[2][2][2];  // [kb][kk][16-byte piece]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int i = l32;
    const int r = 32 * ((i >> 2) & 1) + 16 * kb + 4 * (i >> 3) + (i & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = 4 * kk + 2 * half + p;
        k_off[kb][kk][p] = r * kD8 + ((c ^ k8_swz(r)) & 7) * 16;
      }
  }
  // V^T fragment of block db, piece t: lane j of 16-lane group g reads row
  // 32 (g / 2) + 8 t + j / 2, bytes 8 (j % 2) of chunk 2 db + g % 2, and
  // receives keys 32 (g / 2) + 8 t + [0, 8) of head dimension 32 db + 16 (g % 2) + j
  int v_off[4][4];  // [db][t]
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 32 * (g >> 1) + 8 * t + (j >> 1);
        const int ch = 2 * db + (g & 1);
        v_off[db][t] = r * kD8 + ((ch ^ v8_swz(r)) & 7) * 16 + 8 * (j & 1);
      }
  }

  f32x16_t zero;  // accumulator input of each chain's first product (see header)
#pragma unroll
  for (int r = 0; r < 16; ++r) zero[r] = 0.0f;
  asm volatile("" : "+v"(zero));  // a register block, never an inline constant
  i32x8_t ones;  // e4m3 1.0 in every byte: row sums of the rounded probabilities
#pragma unroll
  for (int w = 0; w < 8; ++w) ones[w] = 0x38383838;
  asm volatile("" : "+v"(ones));

  f32x16_t oacc[4], osum;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) osum[r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;

  auto frag = [&](const char* base, int o0, int o1) {
    const u32x4_t x0 = *(const u32x4_t*)(base + o0);
    const u32x4_t x1 = *(const u32x4_t*)(base + o1);
    i32x8_t f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[w] = (int)x0[w];
      f[4 + w] = (int)x1[w];
    }
    return f;
  };

  const int kt_first = max(t_lo, w_lo / kBC8);  // the wave's first live tile

  auto compute_tile = [&](int kt, const char* kl, const char* vl) {
    const int k0 = kt * kBC8;
    if (!(wave_live && k0 < w_hi && k0 + kBC8 > w_lo)) return;  // nothing allowed for this wave
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the operand stays live until after the product (see header)
      const i32x8_t a0 = frag(kl, k_off[kb][0][0], k_off[kb][0][1]);
      s[kb] = mma8(a0, qf[0], zero);
      asm volatile("" : "+v"(s[kb]) : "v"(a0));
      s[kb] = mma8(frag(kl, k_off[kb][1][0], k_off[kb][1][1]), qf[1], s[kb]);
    }
    // this lane's keys: kj = k0 + 32 half + c, c = 16 kb + r, allowed iff
    // lo <= kj <= hi, i.e. a_lo <= c <= a_hi with per-lane a_lo = lo - k0 -
    // 32 half, a_hi = hi - k0 - 32 half: one compare of the register's
    // constant offset c with a per-lane value and one select per key, per
    // bound the tile crosses
    const bool cut_hi = (k0 + kBC8 > n_k) || (causal && k0 + kBC8 - 1 > wq0 + delta);
    const bool cut_lo = W >= 0 && k0 < wq_last + delta - W;
    if (cut_hi || cut_lo) {
      int hi = n_k - 1, lo = 0;
      if (causal) hi = min(hi, qi + delta);
      if (W >= 0) lo = max(lo, qi + delta - W);
      const int a_hi = hi - k0 - 32 * half, a_lo = lo - k0 - 32 * half;
      if (!cut_lo) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (16 * kb + r > a_hi) s[kb][r] = kNegInf;
      } else if (!cut_hi) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (16 * kb + r < a_lo) s[kb][r] = kNegInf;
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 16 * kb + r;
            if (c > a_hi || c < a_lo) s[kb][r] = kNegInf;
          }
      }
    }
    // the wave's first live tile takes its row max as the reference at once
    // (against -inf every probability would overflow and be recomputed); a
    // row with no allowed key there keeps -inf and goes the slow way below
    if (kt == kt_first) {
      float a4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        a4[c] = fmaxf(fmaxf(fmaxf(s[0][4 * c], s[0][4 * c + 1]), fmaxf(s[0][4 * c + 2], s[0][4 * c + 3])),
                      fmaxf(fmaxf(s[1][4 * c], s[1][4 * c + 1]), fmaxf(s[1][4 * c + 2], s[1][4 * c + 3])));
      const float mt = fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3]));
      m_run = fmaxf(mt, swap_halves(mt)) * c2;
    }
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[kb][r] = exp2_hw(fmaf(s[kb][r], c2, -m_run));
    float rsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) rsum += p[kb][r];
    if (__builtin_amdgcn_ballot_w64(!(rsum <= kLazyBound8)) != 0) {
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      const float m_tile = fmaxf(mt, swap_halves(mt)) * c2;
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_new == m_run ? 1.0f : exp2_hw(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) osum[r] *= alpha;
      m_run = m_new;
      const float m_use = m_run == kNegInf ? 0.0f : m_run;
      rsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb][r] = exp2_hw(fmaf(s[kb][r], c2, -m_use));
          rsum += p[kb][r];
        }
    }
    l_run += rsum;
    // P^T operand: byte j of lane (h, n) = probability of key 32 h + j
    i32x8_t pf;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      pf[w] = (int)pack_fp8x4(p[kb][r], p[kb][r + 1], p[kb][r + 2], p[kb][r + 3]);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x8_t vf;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vl + v_off[db][t]));
        vf[2 * t] = x[0];
        vf[2 * t + 1] = x[1];
      }
      oacc[db] = mma8(vf, pf, oacc[db]);
    }
    osum = mma8(ones, pf, osum);
  };

  if (t_lo < t_hi) {
    issue(t_lo, k_lds0, v_lds0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and the first tile
    __syncthreads();
    for (int kt = t_lo; kt < t_hi; kt += 2) {
      if (kt + 1 < t_hi) issue(kt + 1, k_lds1, v_lds1);
      compute_tile(kt, k_lds0, v_lds0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (kt + 1 < t_hi) {
        if (kt + 2 < t_hi) issue(kt + 2, k_lds0, v_lds0);
        compute_tile(kt + 1, k_lds1, v_lds1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    }
  }

  // epilogue: O = dv * u / (sum of the rounded probabilities), lse from the
  // unrounded sum
  const float l_tot = l_run + swap_halves(l_run);
  const float lr_tot = osum[0];
  if (qi < n_q) {
    const float inv = lr_tot > 0.0f ? vscale / lr_tot : 0.0f;
    uint16_t* op = og + (long long)qi * row_bytes;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + half * 4;
        u32x2_t pr;
        pr[0] = pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
        pr[1] = pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
        *(u32x2_t*)(op + d) = pr;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[(long long)bh * n_q + qi] = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8LaunchArgs& p, hipStream_t stream) {
  const long long bh = (long long)p.batch * p.heads;
  if (bh <= 0 || p.seqlen_q <= 0) return hipSuccess;
  Fp8Args a;
  a.q = (const uint8_t*)p.q;
  a.k = (const uint8_t*)p.k;
  a.v = (const uint8_t*)p.v;
  a.o = (uint16_t*)p.o;
  a.lse = p.lse;
  a.dq = p.descale_q;
  a.dk = p.descale_k;
  a.dv = p.descale_v;
  a.batch = p.batch;
  a.heads = p.heads;
  a.seqlen_q = p.seqlen_q;
  a.seqlen_k = p.seqlen_k;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.window_left = p.window_left < 0 ? -1 : p.window_left;
  const long long grid = bh * ceil_div(p.seqlen_q, kRows8);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3((unsigned)grid), dim3(kThreads8), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
