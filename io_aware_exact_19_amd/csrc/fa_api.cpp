// C ABI of libfa.so: argument checks, then launches on the caller's stream.
// Every check runs on the host before any HIP call, so a rejected call has
// touched neither the device nor the stream.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Head dims the operation is defined for here: 64 and 128.  Any other value
// is an invalid argument, not a missing build.
bool head_dim_valid(int d) { return d == 64 || d == 128; }

// A left window of seqlen_k or more keys admits every key of every row (the
// bound i + delta - W is then <= n_k - 1 - W < 0 for every row i), so it is
// the same as no window.  Mapping it to -1 here keeps the kernels' int32
// bound q0 + delta - W from overflowing for W near INT_MAX.
int effective_window(int window_left, int seqlen_k) {
  return window_left < 0 || window_left >= seqlen_k ? -1 : window_left;
}

int fwd_common(bool fp32, const void* q, const void* k, const void* v, void* o, float* lse,
               int batch, int heads, int seqlen_q, int seqlen_k, int d, float scale, int causal,
               int window_left, const int* cu_q, const int* cu_k, void* stream,
               const int* seqlens_k = nullptr) {
  if (batch < 0 || heads < 0 || seqlen_q < 0 || seqlen_k < 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_valid(d)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if ((cu_q == nullptr) != (cu_k == nullptr)) return FA_ERR_INVALID_ARG;
  if (fp32 && cu_q != nullptr) return FA_ERR_UNSUPPORTED;
  if (batch == 0 || heads == 0 || seqlen_q == 0) return FA_OK;  // nothing to compute
  if (q == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  // with no keys at all (seqlen_k == 0, dense) k and v are never read and may be NULL
  if ((k == nullptr || v == nullptr) && !(seqlen_k == 0 && cu_q == nullptr))
    return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return FA_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (cu_q != nullptr && (!aligned(cu_q, 4) || !aligned(cu_k, 4))) return FA_ERR_INVALID_ARG;
  if (seqlens_k != nullptr && !aligned(seqlens_k, 4)) return FA_ERR_INVALID_ARG;
  // the grid has batch * heads * ceil(seqlen_q / 128) workgroups
  const long long grid = (long long)batch * heads * ((seqlen_q + 127) / 128);
  if (grid > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;

  // K/V rows are addressed with 32-bit byte offsets inside windows of
  // seg_rows rows; one 64-row tile must fit a window
  const unsigned long long row_bytes = (unsigned long long)heads * d * (fp32 ? 4 : 2);
  const unsigned long long win = 0xFFFFFFFFull / row_bytes;
  if (win < 64) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.seg_rows = (int)((win > (1ull << 30) ? (1ull << 30) : win) & ~63ull);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = batch;
  a.heads = heads;
  a.seqlen_q = seqlen_q;
  a.seqlen_k = seqlen_k;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.causal = causal;
  a.window_left = effective_window(window_left, seqlen_k);
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.seqlens_k = seqlens_k;
  a.kv_rows = seqlen_k;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fp32 ? fa::launch_fwd_fp32(a, d, s) : fa::launch_fwd_bf16(a, d, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int heads,
           int seqlen_q, int seqlen_k, int d, float scale, int causal, int window_left,
           const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream) {
  return fwd_common(false, q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, d, scale, causal,
                    window_left, cu_seqlens_q, cu_seqlens_k, stream);
}

int fa_fwd_fp32(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                int heads, int seqlen_q, int seqlen_k, int d, float scale, int causal,
                int window_left, const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream) {
  return fwd_common(true, q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, d, scale, causal,
                    window_left, cu_seqlens_q, cu_seqlens_k, stream);
}

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k,
                   void* o, float* lse, int batch, int heads, int seqlen_q, int max_len, int d,
                   float scale, int causal, int window_left, void* stream) {
  if (seqlens_k == nullptr) return FA_ERR_INVALID_ARG;
  if (batch > 0 && heads > 0 && seqlen_q > 0 && max_len <= 0) return FA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) {
    if (batch > 0 && heads > 0 && seqlen_q > 0) return FA_ERR_INVALID_ARG;
  }
  return fwd_common(false, q, k_cache, v_cache, o, lse, batch, heads, seqlen_q, max_len, d, scale,
                    causal, window_left, nullptr, nullptr, stream, seqlens_k);
}

size_t fa_bwd_workspace_size(int batch, int heads, int seqlen_q) {
  if (batch <= 0 || heads <= 0 || seqlen_q <= 0) return 0;
  return 2 * (size_t)batch * heads * seqlen_q * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int seqlen_q,
           int seqlen_k, int d, float scale, int causal, int window_left, void* workspace,
           size_t workspace_bytes, void* stream) {
  if (batch < 0 || heads < 0 || seqlen_q < 0 || seqlen_k < 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_valid(d)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (batch == 0 || heads == 0 || (seqlen_q == 0 && seqlen_k == 0)) return FA_OK;
  const bool rows = seqlen_q > 0, keys = seqlen_k > 0;
  if (rows && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr))
    return FA_ERR_INVALID_ARG;
  if (keys && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_size(batch, heads, seqlen_q);
  if (rows && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return FA_ERR_WORKSPACE;
  // each workgroup addresses 128 rows of one head with 32-bit offsets
  const unsigned long long row_bytes = (unsigned long long)heads * d * 2;
  if (row_bytes * 128 >= 0x80000000ull) return FA_ERR_UNSUPPORTED;
  const long long g = (long long)batch * heads * ((seqlen_q > seqlen_k ? seqlen_q : seqlen_k) + 127) / 128;
  if (g > 0x7fffffffLL || (long long)batch * heads * seqlen_q > 0x7fffffffLL * 256LL)
    return FA_ERR_UNSUPPORTED;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws_nd = static_cast<float*>(workspace);
  a.ws_nl = rows ? static_cast<float*>(workspace) + (size_t)batch * heads * seqlen_q : nullptr;
  a.batch = batch;
  a.heads = heads;
  a.seqlen_q = seqlen_q;
  a.seqlen_k = seqlen_k;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.causal = causal;
  a.window_left = effective_window(window_left, seqlen_k);
  const hipError_t e = fa::launch_bwd(a, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_workspace_size(int batch, int heads, int max_len, int d, int chunk) {
  if (batch <= 0 || heads <= 0 || max_len <= 0 || d <= 0 || chunk <= 0) return 0;
  const int max_chunks = (max_len + chunk - 1) / chunk;
  const size_t lse_off = fa::decode_ws_lse_offset(batch, heads, max_chunks, d);
  return lse_off + (size_t)batch * heads * max_chunks * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by fa_decode and fa_decode_noalloc; fills everything of `a`
// but the workspace pointers.  need = the workspace bytes of the call.
int decode_common(const void* q, const void* k_cache, const void* v_cache,
                  const int* seqlens_k, void* o, float* lse, int batch, int heads, int max_len,
                  int d, float scale, int chunk, fa::DecodeArgs& a, size_t& need,
                  size_t& lse_off) {
  if (batch < 0 || heads < 0 || max_len < 0 || chunk <= 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_valid(d)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (chunk != 64 && chunk != 128 && chunk != 256 && chunk != 512) return FA_ERR_UNSUPPORTED;
  if (batch == 0 || heads == 0) return FA_OK;
  if (max_len == 0) return FA_ERR_INVALID_ARG;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || seqlens_k == nullptr ||
      o == nullptr)
    return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(seqlens_k, 4))
    return FA_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const int max_chunks = (max_len + chunk - 1) / chunk;
  if ((long long)batch * heads * max_chunks > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  if ((long long)chunk * heads * d * 2 >= 0x80000000LL) return FA_ERR_UNSUPPORTED;
  need = fa_decode_workspace_size(batch, heads, max_len, d, chunk);
  lse_off = fa::decode_ws_lse_offset(batch, heads, max_chunks, d);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  a.ws_o = nullptr;
  a.ws_lse = nullptr;
  a.batch = batch;
  a.heads = heads;
  a.max_len = max_len;
  a.max_chunks = max_chunks;
  a.chunk = chunk;
  a.scale_log2 = scale * 1.4426950408889634f;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k,
              void* o, float* lse, int batch, int heads, int max_len, int d, float scale,
              int chunk, void* workspace, size_t workspace_bytes, void* stream) {
  fa::DecodeArgs a;
  size_t need = 0, lse_off = 0;
  const int st = decode_common(q, k_cache, v_cache, seqlens_k, o, lse, batch, heads, max_len, d,
                               scale, chunk, a, need, lse_off);
  if (st != FA_OK || batch == 0 || heads == 0) return st;
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return FA_ERR_WORKSPACE;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off);
  const hipError_t e = fa::launch_decode(a, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int* seqlens_k, void* o, float* lse, int batch, int heads,
                      int max_len, int d, float scale, int chunk, void* stream) {
  fa::DecodeArgs a;
  size_t need = 0, lse_off = 0;
  const int st = decode_common(q, k_cache, v_cache, seqlens_k, o, lse, batch, heads, max_len, d,
                               scale, chunk, a, need, lse_off);
  if (st != FA_OK || batch == 0 || heads == 0) return st;
  if (need > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
  const hipError_t e =
      fa::launch_decode_scratch(a, d, lse_off, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const float* descale_q, const float* descale_k, const float* descale_v, int batch,
               int heads, int seqlen_q, int seqlen_k, int d, float scale, int causal,
               int window_left, void* stream) {
  if (batch < 0 || heads < 0 || seqlen_q < 0 || seqlen_k < 0) return FA_ERR_INVALID_ARG;
  if (!head_dim_valid(d)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;  // d = 64 is valid but has no fp8 kernel
  if (batch == 0 || heads == 0 || seqlen_q == 0) return FA_OK;
  if (q == nullptr || o == nullptr || descale_q == nullptr || descale_k == nullptr ||
      descale_v == nullptr)
    return FA_ERR_INVALID_ARG;
  if (seqlen_k > 0 && (k == nullptr || v == nullptr)) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4))
    return FA_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  // 32-bit offsets: 64 key rows of K or V and 32 query rows stay below 4 GiB
  const unsigned long long row_bytes = (unsigned long long)heads * d;
  if (row_bytes * 64 >= 0x100000000ull) return FA_ERR_UNSUPPORTED;
  const long long grid = (long long)batch * heads * ((seqlen_q + 127) / 128);
  if (grid > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;

  fa::Fp8LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.descale_q = descale_q;
  a.descale_k = descale_k;
  a.descale_v = descale_v;
  a.batch = batch;
  a.heads = heads;
  a.seqlen_q = seqlen_q;
  a.seqlen_k = seqlen_k;
  a.scale = scale;
  a.causal = causal;
  a.window_left = effective_window(window_left, seqlen_k);
  const hipError_t e = fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: combination not built";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
