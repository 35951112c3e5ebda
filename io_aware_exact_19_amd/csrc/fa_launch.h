// Internal interface between the C ABI (fa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int batch;
  int heads;
  int seqlen_q;  // dense: length; varlen: maximum length (grid sizing)
  int seqlen_k;
  float scale_log2;  // scale * log2(e): scores are kept in base 2
  int causal;
  int window_left;
  const int* cu_q;  // varlen offsets, NULL for dense
  const int* cu_k;
  int seg_rows;     // key rows one 32-bit-offset buffer window covers (multiple of 64)
  const int* seqlens_k;  // KV-cache mode: keys of sequence b are rows [0, seqlens_k[b]) of
  int kv_rows;           // its kv_rows-row cache block; NULL otherwise
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;
  void* o;
  float* lse;
  float* ws_o;    // [batch, heads, max_chunks, d] fp32 normalised chunk outputs
  float* ws_lse;  // [batch, heads, max_chunks] fp32 chunk log2-sum-exp2
  int batch;
  int heads;
  int max_len;
  int max_chunks;
  int chunk;
  float scale_log2;
};

// Byte offset of the chunk lse array inside the decode workspace.
inline size_t decode_ws_lse_offset(int batch, int heads, int max_chunks, int d) {
  const size_t o_bytes = (size_t)batch * heads * max_chunks * d * sizeof(float);
  return (o_bytes + 255) & ~(size_t)255;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_fp32(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, hipStream_t stream);

// Size of the static device array that holds the chunk states of the
// allocation-free decode entry point (one array per GPU, fa_decode.hip).
constexpr size_t kDecodeScratchBytes = (size_t)80 << 20;

// launch_decode with ws_o / ws_lse placed in that array on the stream's GPU
// (the caller has checked that the workspace size fits); lse_off is the byte
// offset of the chunk lse part.
hipError_t launch_decode_scratch(DecodeArgs a, int d, size_t lse_off, hipStream_t stream);

struct BwdArgs {
  const void* q;       // [batch, seqlen_q, heads, d] bf16
  const void* k;       // [batch, seqlen_k, heads, d] bf16
  const void* v;
  const void* o;       // forward output, layout of q
  const void* dout;    // gradient of the loss with respect to o
  const float* lse;    // [batch, heads, seqlen_q] natural-log row log-sum-exp
  void* dq;
  void* dk;
  void* dv;
  float* ws_nd;        // [batch, heads, seqlen_q] -rowsum(dO o O)
  float* ws_nl;        // [batch, heads, seqlen_q] -lse / scale (score units)
  int batch;
  int heads;
  int seqlen_q;
  int seqlen_k;
  float scale;
  float scale_log2;
  int causal;
  int window_left;
};

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream);

struct Fp8LaunchArgs {
  const void* q;             // [batch, seqlen_q, heads, 128] e4m3
  const void* k;             // [batch, seqlen_k, heads, 128] e4m3
  const void* v;             // [batch, seqlen_k, heads, 128] e4m3
  void* o;                   // [batch, seqlen_q, heads, 128] bf16
  float* lse;                // [batch, heads, seqlen_q] or null
  const float* descale_q;    // [batch * heads]
  const float* descale_k;
  const float* descale_v;
  int batch, heads, seqlen_q, seqlen_k;
  float scale;
  int causal, window_left;
};

hipError_t launch_fwd_fp8(const Fp8LaunchArgs& p, hipStream_t stream);

}  // namespace fa
