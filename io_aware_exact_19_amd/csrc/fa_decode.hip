// Split-KV attention decode for gfx950: one new query per sequence against
// its KV cache.
//
// Decode reads the whole cache once per token and does about one FLOP per
// byte, so it is bound by HBM bandwidth, not by the matrix cores ("How
// FlashAttention accelerates Transformer attention with IO-aware tiling"
// (wiblog.cn), section "Training, prefill and decode" and its table 1).  The
// design therefore maximises bytes in flight and never touches the cache
// past each sequence's length:
//
//  * split kernel: one workgroup per (sequence, chunk of keys, head).  Each
//    thread issues all of its 16-byte K and V loads for the chunk up front,
//    then computes the chunk's scores (fp32 dot products, base-2 domain with
//    log2(e) folded into the scale), the chunk max, the exponentials, the
//    exp-sum and the probability-weighted V sum, and writes the chunk's
//    normalised output and log2-sum-exp2 to the workspace.  This is the
//    per-row recurrence of "FlashAttention" (aiwiki.page), section "Tiling
//    and online normalisation", over one chunk (the key tiling of "From
//    Online Softmax to FlashAttention" (cloud.tencent.cn), section 4).
//  * combine kernel: one wave per (sequence, head) merges the chunk states
//    with the same rescale: weights 2^(lse_c - max), output = weighted mean.
//
// Consecutive workgroups take consecutive heads of the same (sequence,
// chunk), so concurrently running workgroups read neighbouring 256-byte
// pieces of the same 8 KB cache rows.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// Sum over aligned groups of N lanes (N in {8, 16}) with DPP row permutes.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)); // half-row mirror
  if constexpr (N == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true)); // row mirror
  return x;
}

template <int D, int CHUNK>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int kLpk = D / 8;          // lanes per key row (16 bytes each)
  constexpr int kKpi = 64 / kLpk;      // keys per wave per load instruction
  constexpr int kKpw = CHUNK / 4;      // keys per wave
  constexpr int kIt = kKpw / kKpi;     // loads per thread per tensor
  static_assert(kKpw % kKpi == 0, "chunk must split over the wave");
  __shared__ float s_max[4];
  __shared__ float s_sum[4];
  __shared__ float s_o[4][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads;
  const int h = blockIdx.x % H;
  const int bc = blockIdx.x / H;
  const int c = bc % a.max_chunks;
  const int b = bc / a.max_chunks;
  const int L = min(max(a.seqlens[b], 0), a.max_len);
  if (c * CHUNK >= L) return;  // chunk past this sequence's length

  const int sub = lane / kLpk, dl = lane % kLpk;
  const long long rs = (long long)H * D;
  const uint16_t* kp = (const uint16_t*)a.k + ((long long)b * a.max_len * H + h) * D + dl * 8;
  const uint16_t* vp = (const uint16_t*)a.v + ((long long)b * a.max_len * H + h) * D + dl * 8;
  const int key0 = c * CHUNK + wave * kKpw + sub;

  u32x4_t kr[kIt], vr[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int key = key0 + it * kKpi;
    kr[it] = key < L ? *(const u32x4_t*)(kp + (long long)key * rs) : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int key = key0 + it * kKpi;
    vr[it] = key < L ? *(const u32x4_t*)(vp + (long long)key * rs) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // query slice of this lane, scaled into the base-2 domain
  float qf[8];
  {
    const u32x4_t qw = *(const u32x4_t*)((const uint16_t*)a.q + ((long long)b * H + h) * D + dl * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[2 * j] = bf16_lo(qw[j]) * a.scale_log2;
      qf[2 * j + 1] = bf16_hi(qw[j]) * a.scale_log2;
    }
  }

  // scores of this lane's keys (every lane of a key group ends with the sum)
  float s[kIt];
  float mx = kNegInf;
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      part = fmaf(qf[2 * j], bf16_lo(kr[it][j]), part);
      part = fmaf(qf[2 * j + 1], bf16_hi(kr[it][j]), part);
    }
    part = group_sum<kLpk>(part);
    s[it] = (key0 + it * kKpi) < L ? part : kNegInf;
    mx = fmaxf(mx, s[it]);
  }
  // max over the key groups of the wave, then over the 4 waves
#pragma unroll
  for (int off = kLpk; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));  // finite: >= 1 key

  float l = 0.0f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.0f;
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const float p = exp2_hw(s[it] - m);
    l += p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = fmaf(p, bf16_lo(vr[it][j]), o[2 * j]);
      o[2 * j + 1] = fmaf(p, bf16_hi(vr[it][j]), o[2 * j + 1]);
    }
  }
#pragma unroll
  for (int off = kLpk; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] += __shfl_xor(o[j], off, 64);
  }
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[wave][dl * 8 + j] = o[j];
    if (dl == 0) s_sum[wave] = l;
  }
  __syncthreads();
  const float lt = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
  const long long slot = ((long long)b * H + h) * a.max_chunks + c;
  if (tid < D) {
    const float acc = s_o[0][tid] + s_o[1][tid] + s_o[2][tid] + s_o[3][tid];
    a.ws_o[slot * D + tid] = acc / lt;
  }
  if (tid == 0) a.ws_lse[slot] = m + log2_hw(lt);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  constexpr int kPer = D / 64;  // output dims per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= a.batch * a.heads) return;
  const int b = idx / a.heads, h = idx - b * a.heads;
  const int L = min(max(a.seqlens[b], 0), a.max_len);
  const int n = (L + a.chunk - 1) / a.chunk;
  const float* lp = a.ws_lse + (long long)idx * a.max_chunks;
  const float* op = a.ws_o + (long long)idx * a.max_chunks * D;

  float mx = kNegInf;
  for (int c = lane; c < n; c += 64) mx = fmaxf(mx, lp[c]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));

  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.0f;
  float wsum = 0.0f;
  for (int c = 0; c < n; ++c) {
    const float wgt = exp2_hw(lp[c] - mx);
    wsum += wgt;
#pragma unroll
    for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wgt, op[(long long)c * D + lane * kPer + j], acc[j]);
  }
  const float inv = n > 0 ? 1.0f / wsum : 0.0f;
  uint16_t* o = (uint16_t*)a.o + ((long long)b * a.heads + h) * D + lane * kPer;
  if constexpr (kPer == 2) {
    *(uint32_t*)o = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    union { __bf16 v; uint16_t u; } cv;
    cv.v = (__bf16)(acc[0] * inv);
    *o = cv.u;
  }
  if (a.lse != nullptr && lane == 0)
    a.lse[idx] = n > 0 ? (mx + log2_hw(wsum)) * kLn2 : kNegInf;
}

template <int D, int CHUNK>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const long long g1 = (long long)a.batch * a.max_chunks * a.heads;
  if (g1 > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g1 > 0) {
    hipLaunchKernelGGL((decode_split_kernel<D, CHUNK>), dim3((unsigned)g1), dim3(kThreads), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long g2 = ((long long)a.batch * a.heads + 3) / 4;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)g2), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.chunk) {
    case 64: return launch_t<D, 64>(a, stream);
    case 128: return launch_t<D, 128>(a, stream);
    case 256: return launch_t<D, 256>(a, stream);
    case 512: return launch_t<D, 512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_d<128>(a, stream);
  if (d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
