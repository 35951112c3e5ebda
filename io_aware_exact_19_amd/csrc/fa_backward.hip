// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale Q K^T) V for
// an output gradient dO, recomputing the probabilities from the row
// log-sum-exp the forward pass emits instead of storing them -- the reason
// the forward keeps lse ("FlashAttention" (aiwiki.page), section "Training
// and computational complexity").  With P = exp(scale Q K^T - lse) (zero on
// masked pairs) the gradients are the chain rule through the softmax:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id (= rowsum(P o dP)),
//   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, no atomics (every output element has one writer), dq first
// (dq in fa_backward_dq.hip, dkdv here, shared helpers in fa_backward.h):
//  * dq: one workgroup per (batch, head, 128 query rows); each wave owns 32
//    rows (Q and dO fragments in registers) while 64-key tiles of K and V
//    stream through the ring: S^T = K Q^T, dP^T = V dO^T, dS^T on the VALU,
//    then dQ^T += K^T dS^T.  It also reads its rows of O in the dO fragment
//    layout, forms D_i once the loop's first step (score products only) is
//    issued, and writes -D_i and -lse_i / scale of each row into the
//    workspace for the dkdv kernel.
//  * dkdv: one workgroup of 4 waves (one per SIMD) per (batch, head, 128
//    keys), or at d = 128 with more such items than CUs one persistent
//    workgroup per CU walking several of them; each wave owns 32 keys and
//    keeps their K and V fragments in registers while 64-row tiles of Q, dO,
//    -lse/scale, -D stream through a ring of LDS slots.  A persistent
//    workgroup queues the next item's first two tiles in the two loads after
//    the current item's last tile and its K, V once the current item's score
//    products are done.  -D and -lse / scale seed the dP and S accumulators, so
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
#include "fa_backward.h"

namespace fa {
namespace {

// ---------------------------------------------------------------- dK, dV
// Work items: (batch, head, 128-key tile).  On small grids each workgroup
// runs one item (bwd_unit).  Larger launches are persistent (see
// launch_bwd_dkdv_t): one workgroup per CU, grid a multiple of 8, and XCD x
// walks the items of the heads x, x + 8, ... in rounds, local workgroup w
// taking item r * G8 + w of the XCD's list in even rounds and
// r * G8 + G8 - 1 - w in odd ones.  Under a mask the list runs in rank order
// (rank 0 = the tile with the most query rows, every head's tile of one rank
// before the next rank), so long and short items of consecutive rounds pair
// up; without one every item costs the same and the list is head by head,
// so the tiles that run together share their head's Q and dO in the L2.
__device__ __forceinline__ bool dkdv_item(int r, int nbh, int nkt, int order, int& bh, int& kt) {
  if ((long long)gridDim.x >= (long long)nbh * nkt) {
    if (r > 0) return false;
    bwd_unit(nbh, nkt, order, bh, kt);
    return true;
  }
  const int g8 = (int)gridDim.x >> 3, wb = (int)blockIdx.x >> 3, x = (int)blockIdx.x & 7;
  const int hx = nbh >> 3;
  const int k = r * g8 + ((r & 1) ? g8 - 1 - wb : wb);
  if (k >= hx * nkt) return false;
  if (order == 0) {
    const int j = k / nkt;
    bh = x + 8 * j;
    kt = k - j * nkt;
  } else {
    const int rank = k / hx;
    bh = x + 8 * (k - rank * hx);
    kt = order < 0 ? nkt - 1 - rank : rank;
  }
  return true;
}

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
  const int nkt = ceil_div(n_k, kUnit), nbh = a.batch * H;
  const int order = causal ? 1 : (W >= 0 ? -1 : 0);
  const long long rs = (long long)H * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const float c2 = a.scale_log2;

  // one item: its (batch, head), this wave's first key, and the 64-row tiles
  // [t_lo, t_lo + nt) of query rows that can see one of its keys
  struct Item {
    int b, h, wk0, t_lo, nt;
  };
  auto make_item = [&](int bh_, int kt_) {
    Item it;
    it.h = bh_ % H;
    it.b = bh_ / H;
    const int k0 = kt_ * kUnit;
    it.wk0 = k0 + wave * kWaveRows;
    int q_lo = 0, q_hi = n_q;
    if (causal) q_lo = max(q_lo, k0 - delta);
    if (W >= 0) q_hi = min(q_hi, k0 + kUnit - delta + W);
    it.t_lo = q_lo / kTile;
    it.nt = q_hi > q_lo ? ceil_div(q_hi, kTile) - it.t_lo : 0;
    return it;
  };
  int r_item = 0, bh_n = 0, kt_n = 0;
  if (!dkdv_item(0, nbh, nkt, order, bh_n, kt_n)) return;
  Item cur = make_item(bh_n, kt_n), nxt = cur;
  bool has_next = false;
  int gbase = 0;  // ring index of the current item's first tile

  // K, V of this wave's 32 keys as B operands
  auto owner = [&](const Item& it, bf16x8_t (&kx)[D / 16], bf16x8_t (&vx)[D / 16]) {
    const long long base = ((long long)it.b * n_k * H + it.h) * D;
    load_owner<D>(kx, (const uint16_t*)a.k + base, rs, it.wk0, n_k, lane);
    load_owner<D>(vx, (const uint16_t*)a.v + base, rs, it.wk0, n_k, lane);
  };
  bf16x8_t kf[D / 16], vf[D / 16];
  owner(cur, kf, vf);

  f32x16_t dk[D / 32], dv[D / 32];  // dK^T, dV^T: [d][key], lane = key

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
  auto slot = [&](int g) { return ring + (g & (kRing - 1)) * kSlot; };
  // the ring's LDS byte address as an integer: the DMA destinations are
  // computed from it, without casting a slot pointer chosen at run time
  const uint32_t ring_lds = lds_addr(ring);
  // tile u of item it into ring slot g; u outside [0, it.nt) gives
  // descriptors of size 0 (the loads write zeros into a free slot)
  auto dma_tile = [&](const Item& it, int u, int g) {
    DmaTile t;
    const bool live = u >= 0 && u < it.nt;
    const int r0 = live ? (it.t_lo + u) * kTile : 0;
    const uint32_t rows = live ? (uint32_t)min(kTile, n_q - r0) : 0u;
    const long long qb = ((long long)it.b * n_q * H + it.h) * D + (long long)r0 * rs;
    const long long vb = ((long long)it.b * H + it.h) * n_q + r0;
    t.x = rsrc_of((const uint16_t*)a.q + qb, rows * row_bytes);
    t.y = rsrc_of((const uint16_t*)a.dout + qb, rows * row_bytes);
    // waves 0, 2 load -lse/scale, waves 1, 3 load -D (the same values twice)
    t.vec = rsrc_of(((wave & 1) ? a.ws_nd : a.ws_nl) + vb, rows * 4);
    t.lds = ring_lds + (uint32_t)(g & (kRing - 1)) * kSlot;
    return t;
  };
  // the two loads that follow the current item's last tile fetch the next
  // item's first two tiles, so they are in LDS when that item starts
  auto dma_setup = [&](int u) {
    if (u < cur.nt || !has_next) return dma_tile(cur, u, gbase + u);
    return dma_tile(nxt, u - cur.nt, gbase + u);
  };
  auto dma_piece = [&](const DmaTile& t, int k) {
    if (k < 2) {
      dma_group(k == 0 ? t.x : t.y, t.lds + k * T::kBytes + wave * T::kLoads * 1024);
    } else {
      dma_b32(t.vec, (uint32_t)lane * 4, t.lds + 2 * T::kBytes + (wave & 1) * T::kVec);
    }
  };

  const FragOffsets<D> fo(lane);
  f32x16_t sacc[2], dpacc[2];  // [block parity]: S and dP of one 32-row block
  bf16x8_t pf[2][2], sf[2][2];  // [block parity][16-row slice]: P and dS as B operands
  auto block_row0 = [&](int j) { return (cur.t_lo + (j >> 1)) * kTile + kWaveRows * (j & 1); };
  auto block_masked = [&](int j) {
    const int r0 = block_row0(j);
    return (causal && cur.wk0 + kWaveRows - 1 > r0 + delta) ||
           (W >= 0 && cur.wk0 < r0 + kWaveRows - 1 + delta - W);
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
    const char* x1 = slot(gbase + ((j + 1) >> 1)) + (1 - p) * kWaveRows * T::kRowB;
    const char* x2 = slot(gbase + ((j - 1) >> 1)) + (1 - p) * kWaveRows * T::kRowB;

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
      const char* vb =
          slot(gbase + ((j + 1) >> 1)) + 2 * T::kBytes + (kWaveRows * (1 - p) + 8 * half) * 4;
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
      const int w = cur.wk0 + l32 - delta - block_row0(j) - 8 * half;
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

  constexpr Bool<true> y{};
  constexpr Bool<false> n{};
  bool queued = false;  // the current item's first two tiles are already in flight
  for (;;) {
    has_next = dkdv_item(r_item + 1, nbh, nkt, order, bh_n, kt_n);
    if (has_next) nxt = make_item(bh_n, kt_n);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[db][r] = 0.0f;
        dv[db][r] = 0.0f;
      }
    const int nt = cur.nt;
    if (nt > 0) {
      if (!queued) {
        const DmaTile t0 = dma_setup(0), t1 = dma_setup(1);
#pragma unroll
        for (int k = 0; k < kPieces; ++k) dma_piece(t0, k);
#pragma unroll
        for (int k = 0; k < kPieces; ++k) dma_piece(t1, k);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));  // tile 0 has landed
      } else {
        // tiles 0 and 1 were queued during the previous item, before its
        // loads of this item's K, V and its output stores
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
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
      // the score products are done: the next item's K, V go out now,
      // into the same registers
      if (has_next) owner(nxt, kf, vf);
      step(n, y, y, y, Int<1>{}, n, DmaTile{}, 2 * nt - 1);
      step(n, y, n, n, Int<0>{}, n, DmaTile{}, 2 * nt);
    } else {
      // no query row sees these keys: dK = dV = 0
      if (has_next) owner(nxt, kf, vf);
    }

    // lane holds d = 32 db + 8 (r/4) + 4 h + r%4 of its key
    const int key = cur.wk0 + l32;
    if (key < n_k) {
      const long long ob = (((long long)cur.b * n_k + key) * H + cur.h) * D;
      uint16_t* dkp = (uint16_t*)a.dk + ob;
      uint16_t* dvp = (uint16_t*)a.dv + ob;
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
    if (!has_next) break;
    // an item without tiles queued nothing for the next one
    queued = nt > 0;
    gbase += nt;
    cur = nxt;
    ++r_item;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the size-0 loads of the last tiles
}

template <int D>
hipError_t launch_bwd_dkdv_t(const BwdArgs& a, hipStream_t stream) {
  const long long nbh = (long long)a.batch * a.heads;
  long long g = nbh * ceil_div(a.seqlen_k, kUnit);
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g == 0) return hipSuccess;
  // d = 128 (one workgroup per CU): persistent when there are more items
  // than CUs and the heads split evenly over the XCDs
  if (D == 128 && nbh % 8 == 0) {
    const int slots = bwd_slots();
    if (slots >= 8 && g > slots) g = slots;
  }
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)g), dim3(kBThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t stream) {
  if (d != 128 && d != 64) return hipErrorInvalidValue;
  // both grids checked before either kernel runs
  if ((long long)a.batch * a.heads * ceil_div(a.seqlen_k, kUnit) > 0x7fffffffLL ||
      (long long)a.batch * a.heads * ceil_div(a.seqlen_q, kUnit) > 0x7fffffffLL)
    return hipErrorInvalidValue;
  // dq first: it writes the per-row workspace values that dkdv reads
  const hipError_t e = launch_bwd_dq(a, d, stream);
  if (e != hipSuccess) return e;
  return d == 128 ? launch_bwd_dkdv_t<128>(a, stream) : launch_bwd_dkdv_t<64>(a, stream);
}

}  // namespace fa
