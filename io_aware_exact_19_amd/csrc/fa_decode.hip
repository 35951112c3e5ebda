// Split-KV attention decode for gfx950: one new query per sequence against
// its KV cache.
//
// Decode reads the whole cache once per token and does about one FLOP per
// byte, so it is bound by HBM bandwidth, not by the matrix cores ("How
// FlashAttention accelerates Transformer attention with IO-aware tiling"
// (wiblog.cn), section "Training, prefill and decode" and its table 1).  The
// design therefore keeps as many cache bytes in flight as the register file
// allows and never touches the cache past each sequence's length:
//
//  * split kernel: one workgroup of 4 waves per (sequence, chunk of keys,
//    group of heads).  A wave owns D/8-lane groups, one per head (16 bytes of
//    the head's row per lane), so each of its loads reads one contiguous
//    1 KB piece of a key row (4 heads at d = 128, 8 at d = 64).  The wave
//    walks its chunk in steps of kStep keys with two register buffers: the
//    loads of step s+1 (2 * kStep 16-byte loads per lane, nontemporal) are in
//    flight while step s is scored.  Per step it runs the online-softmax
//    update of "FlashAttention" (aiwiki.page), section "Tiling and online
//    normalisation", in the base-2 domain with log2(e) folded into the scale:
//    scores, new running max, rescale of the exp-sum and of the accumulator,
//    then the probability-weighted V sum.  At the end of the chunk it writes
//    the normalised partial output and log2-sum-exp2 to the workspace (the
//    key tiling of "From Online Softmax to FlashAttention" (cloud.tencent.cn),
//    section 4).  Loads use a buffer descriptor that ends at the chunk's last
//    valid key, so rows past the sequence length read as zeros in hardware and
//    their scores are masked to -inf.
//  * combine kernel: one wave per (sequence, head) merges the chunk states
//    with the same rescale: weights 2^(lse_c - max), output = weighted mean.
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

// Chunk states of the allocation-free entry point: one array per GPU, created
// with the code object and held until the process ends.  In host code the
// name `scratch` only stands for the device symbol; its device address comes
// from hipGetSymbolAddress, once per device (decode_scratch_ptr below).
static __device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStep = 16;                // keys per pipeline step
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kNontemporal = 2;          // cache policy of the streaming loads

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

template <int D>
constexpr int heads_per_group() { return kWaves * (64 / (D / 8)); }

template <int D, int CHUNK>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int kLpk = D / 8;            // lanes per head row (16 bytes each)
  constexpr int kHpw = 64 / kLpk;        // heads per wave
  constexpr int kHpg = heads_per_group<D>();
  static_assert(CHUNK % (2 * kStep) == 0, "two pipeline steps per loop trip");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.heads;
  const int n_hg = (H + kHpg - 1) / kHpg;
  const int hg = blockIdx.x % n_hg;
  const int bc = blockIdx.x / n_hg;
  const int c = bc % a.max_chunks;
  const int b = bc / a.max_chunks;
  const int L = min(max(a.seqlens[b], 0), a.max_len);
  const int key0 = c * CHUNK;
  if (key0 >= L) return;  // chunk past this sequence's length
  const int n = min(CHUNK, L - key0);

  const int dl = lane % kLpk;
  const int h = hg * kHpg + wave * kHpw + lane / kLpk;
  const bool hv = h < H;  // lanes of heads past the last one load nothing
  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const long long chunk_elems = ((long long)b * a.max_len + key0) * H * D;
  // The descriptors end at the chunk's last valid key: loads past it return
  // zeros.  Offsets stay below 2^31 (checked by the host), so the offset
  // 2^31 of inactive lanes is always out of range.
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.k + chunk_elems), 0, (uint32_t)n * row_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.v + chunk_elems), 0, (uint32_t)n * row_bytes, kRsrcWord3);
  const uint32_t lane_off = hv ? (uint32_t)(h * D + dl * 8) * 2 : 0x80000000u;

  // query slice of this lane, scaled into the base-2 domain
  float qf[8];
  {
    u32x4_t qw = {0u, 0u, 0u, 0u};
    if (hv) qw = *(const u32x4_t*)((const uint16_t*)a.q + ((long long)b * H + h) * D + dl * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[2 * j] = bf16_lo(qw[j]) * a.scale_log2;
      qf[2 * j + 1] = bf16_hi(qw[j]) * a.scale_log2;
    }
  }

  u32x4_t ka[kStep], va[kStep], kb[kStep], vb[kStep];
  auto load = [&](u32x4_t (&kr)[kStep], u32x4_t (&vr)[kStep], int st) {
    const uint32_t base = lane_off + (uint32_t)(st * kStep) * row_bytes;
#pragma unroll
    for (int i = 0; i < kStep; ++i)
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, base + i * row_bytes, 0, kNontemporal);
#pragma unroll
    for (int i = 0; i < kStep; ++i)
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, base + i * row_bytes, 0, kNontemporal);
  };

  float m = kNegInf, l = 0.0f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.0f;
  // online-softmax update with the keys of step st
  auto update = [&](const u32x4_t (&kr)[kStep], const u32x4_t (&vr)[kStep], int st) {
    float sc[kStep];
    float mx = m;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part = fmaf(qf[2 * j], bf16_lo(kr[i][j]), part);
        part = fmaf(qf[2 * j + 1], bf16_hi(kr[i][j]), part);
      }
      part = group_sum<kLpk>(part);  // every lane of the head's group holds the score
      sc[i] = st * kStep + i < n ? part : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    // the first step holds key 0 of the chunk, so mx is finite from then on
    const float alpha = exp2_hw(m - mx);  // 0 on the first step (m = -inf)
    m = mx;
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= alpha;
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const float p = exp2_hw(sc[i] - mx);
      l += p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = fmaf(p, bf16_lo(vr[i][j]), o[2 * j]);
        o[2 * j + 1] = fmaf(p, bf16_hi(vr[i][j]), o[2 * j + 1]);
      }
    }
  };

  // two register buffers: the loads of the next step are in flight while
  // the current one is scored
  const int steps = (n + kStep - 1) / kStep;
  load(ka, va, 0);
  for (int st = 0; st < steps; st += 2) {
    if (st + 1 < steps) load(kb, vb, st + 1);
    update(ka, va, st);
    if (st + 1 >= steps) break;
    if (st + 2 < steps) load(ka, va, st + 2);
    update(kb, vb, st + 1);
  }

  if (hv) {
    const long long slot = ((long long)b * H + h) * a.max_chunks + c;
    const float inv = 1.0f / l;
    const f32x4_t w0 = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    const f32x4_t w1 = {o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    *(f32x4_t*)(a.ws_o + slot * D + dl * 8) = w0;
    *(f32x4_t*)(a.ws_o + slot * D + dl * 8 + 4) = w1;
    if (dl == 0) a.ws_lse[slot] = m + log2_hw(l);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  constexpr int kPer = D / 64;  // output dims per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int idx = blockIdx.x * kWaves + wave;
  if (idx >= a.batch * a.heads) return;
  const int b = idx / a.heads, h = idx - b * a.heads;
  const int L = min(max(a.seqlens[b], 0), a.max_len);
  const int n = (L + a.chunk - 1) / a.chunk;
  const float* lp = a.ws_lse + (long long)idx * a.max_chunks;
  const float* op = a.ws_o + (long long)idx * a.max_chunks * D + lane * kPer;

  float mx = kNegInf;
  for (int c = lane; c < n; c += 64) mx = fmaxf(mx, lp[c]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));

  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.0f;
  float wsum = 0.0f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    // lane i holds the weight of chunk c0 + i; the loop reads it back per chunk
    const float w_lane = c0 + lane < n ? exp2_hw(lp[c0 + lane] - mx) : 0.0f;
    const int cnt = min(64, n - c0);
    int i = 0;
    for (; i + 8 <= cnt; i += 8) {  // eight chunk rows in flight
      float x[8][kPer];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j) x[u][j] = op[(long long)(c0 + i + u) * D + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), i + u));
        wsum += wgt;
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wgt, x[u][j], acc[j]);
      }
    }
    for (; i < cnt; ++i) {
      const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), i));
      wsum += wgt;
#pragma unroll
      for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wgt, op[(long long)(c0 + i) * D + j], acc[j]);
    }
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
  constexpr int kHpg = heads_per_group<D>();
  // offsets inside one chunk's descriptor, plus the 2^31 of inactive lanes,
  // must stay within 32 bits
  if ((long long)CHUNK * a.heads * D * 2 >= 0x80000000LL) return hipErrorInvalidValue;
  const long long g1 = (long long)a.batch * a.max_chunks * ((a.heads + kHpg - 1) / kHpg);
  if (g1 > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g1 > 0) {
    hipLaunchKernelGGL((decode_split_kernel<D, CHUNK>), dim3((unsigned)g1), dim3(kThreads), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long g2 = ((long long)a.batch * a.heads + kWaves - 1) / kWaves;
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

namespace {

constexpr int kMaxDevices = 256;

// Device address of `scratch` on `dev`, looked up once per device with that
// device current (the previous current device is restored).
hipError_t decode_scratch_ptr(int dev, char** out) {
  static std::mutex mu;
  static char* ptrs[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<char*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_scratch(DecodeArgs a, int d, size_t lse_off, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  char* base = nullptr;
  if ((e = decode_scratch_ptr(dev, &base)) != hipSuccess) return e;
  // every chunk state the combine kernel reads is written by the split kernel
  // of the same call, so the array needs no clearing between calls
  a.ws_o = reinterpret_cast<float*>(base);
  a.ws_lse = reinterpret_cast<float*>(base + lse_off);
  return launch_decode(a, d, stream);
}

}  // namespace fa
