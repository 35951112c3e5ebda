// dQ of the attention backward for gfx950 (the algorithm, the tile layout and
// the pipeline are described in fa_backward.hip).  In its own translation
// unit so that it can be compiled with the matrix products' results in
// architectural VGPRs: its working set fits there, and the score
// accumulators then feed the softmax without a copy out of the accumulation
// registers on every step.
#include "fa_backward.h"

namespace fa {
namespace {

// ---------------------------------------------------------------- dQ
// NW waves per workgroup, 32 query rows each.  Eight (two per SIMD, 256 rows
// sharing each K/V tile) let one wave's waits be filled by the other's work;
// the launcher takes them at d = 128 when that grid still fills every CU.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdArgs a) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int kUnit = NW * kWaveRows;  // query rows of one workgroup
  // operand fragments read ahead of their product: one fewer with two waves
  // per SIMD (256 registers each), whose partner covers the LDS latency
  constexpr int kLookQ = NW == 8 ? 2 : kLook;
  using T = BTile<D, NW>;
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
    t.lds = lds_addr(slot(u));
    return t;
  };
  auto dma_piece = [&](const DmaTile& t, int k) {
    dma_group(k == 0 ? t.x : t.y, t.lds + k * T::kBytes + wave * T::kLoads * 1024);
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
      bf16x8_t fq[kLookQ + 1];
#pragma unroll
      for (int i = 0; i < kLookQ && i < kN; ++i) fq[i] = fetch(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kLookQ < kN) fq[(i + kLookQ) % (kLookQ + 1)] = fetch(i + kLookQ);
        product(i, fq[i % (kLookQ + 1)]);
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
    // O was requested before tile 0, so it has landed too
    row_terms();
    step(y, n, n, n, Int<1>{}, n, DmaTile{}, -1);
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

template <int D, int NW>
hipError_t launch_bwd_dq_t(const BwdArgs& a, hipStream_t stream) {
  const long long g = (long long)a.batch * a.heads * ceil_div(a.seqlen_q, NW * kWaveRows);
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)g), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) {
    // eight waves only when their grid (one workgroup per CU) fills the chip:
    // on smaller grids four-wave workgroups reach twice as many CUs.  Under a
    // mask the workgroups differ in length, and the longest-first order needs
    // at least two rounds of them to even the CUs out.
    const long long g8 = (long long)a.batch * a.heads * ceil_div(a.seqlen_q, 8 * kWaveRows);
    const int cus = cu_count();
    const int rounds = (a.causal || a.window_left >= 0) ? 2 : 1;
    return cus > 0 && g8 >= (long long)rounds * cus ? launch_bwd_dq_t<128, 8>(a, stream)
                                                    : launch_bwd_dq_t<128, 4>(a, stream);
  }
  if (d == 64) return launch_bwd_dq_t<64, 4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
