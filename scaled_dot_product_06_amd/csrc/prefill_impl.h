// Prefill: tiled online-softmax attention over query blocks (gfx950 MFMA).
//
// One workgroup = NW wavefronts = `heads` query heads of one key/value group x
// (NW / heads) x MF consecutive query rows. The workgroup walks the key axis in
// tiles of BN keys, staging each K and V tile once in LDS for all its
// wavefronts. Each wavefront keeps its MF query rows' Q fragment, running
// maximum, running sum and output accumulator in registers for the whole walk
// (the per-tile recurrence of lattice-inference "src/attention/flash.rs",
// run_tiled_attention_head). Scores are computed transposed, S^T = K Q^T, so a
// lane's accumulators all belong to one query row: the row maximum needs one
// cross-lane exchange and the output rescale is a per-lane scalar. P goes back
// into the MFMA as the B operand of O^T = V^T P^T; the V^T operand is read
// from the row-major V tile with LDS transpose reads.
//
// Causal masking is bottom-right aligned (nuvec-core "tests/fast.rs", direct
// formula test): row i sees keys j <= i + Lk - Lq. Workgroups stop at their
// last visible key; only tiles that cross a row's last key are masked per
// element. Late (long) query blocks are dispatched first.
//
// ADD instantiations read an additive mask (nuvec-core "tests/fast.rs",
// attention_kernels_match_the_fallback): each lane fetches its row's mask
// values for the next tile together with that tile's K/V (a whole step ahead,
// kept as packed 16-bit values), and adds them (in base 2) to the scaled
// scores. Q, K and V are read through element
// strides (batch, head, row), so views such as a transposed [B, L, H, D]
// array or a slice of a longer cache need no copy.
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int MF, int D, int DV, int BN, int NW>
struct PrefillCfg {
  static constexpr int KW = Mfma<MF>::KW, ACC = Mfma<MF>::ACC, KG = Mfma<MF>::KG;
  static constexpr int DVP = (DV + MF - 1) / MF * MF;  // V columns padded to whole MFMA tiles
  static constexpr int KST = D + 8;                      // LDS row strides (elements)
  static constexpr int VST = DVP + 16;
  static constexpr int NQC = D / KW;
  static constexpr int NSB = BN / MF;
  static constexpr int NPV = BN / KW;
  static constexpr int NDB = DVP / MF;
  static constexpr int NT = NW * 64;
  static constexpr int KCH = BN * D / 8, VCH = BN * DV / 8;  // 16-byte chunks per tile
  static constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT;
  static constexpr int LDS_ELEMS = BN * KST + BN * VST;
  static_assert(D % KW == 0, "head size must be a whole number of MFMA k-steps");
  static_assert(BN % MF == 0 && BN % KW == 0, "tile must hold whole MFMA blocks");
};

template <class E, int MF, int D, int DV, int BN, int NW, bool ADD>
__global__ void __launch_bounds__(NW * 64) prefill_kernel(FwdArgs a) {
  using C = PrefillCfg<MF, D, DV, BN, NW>;
  using acc_t = typename Mfma<MF>::acc_t;
  constexpr int ACC = C::ACC;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* Ks = lds;
  uint16_t* Vs = lds + BN * C::KST;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane % MF;
  const int kg = lane / MF;

  const int heads = a.Hq * a.B / a.head_blocks;   // query heads per workgroup
  const int wph = NW / heads;                      // wavefronts per head
  const int bm = wph * MF;                         // query rows per head per workgroup
  int hb, qb;
  prefill_item((int)blockIdx.x, a.head_blocks, a.nqb, a.group / heads, hb, qb);
  const int groups_per_b = a.Hq / heads;
  const int b = hb / groups_per_b;
  const int h0 = (hb % groups_per_b) * heads;
  const int hkv = h0 / a.group;
  const int h = h0 + w / wph;
  const int wi0 = qb * bm + (w % wph) * MF;
  const int iq = wi0 + col;
  const int shift = a.Lk - a.Lq;

  // keys the workgroup needs: up to its last row's causal limit and, with a
  // sliding window, from its first row's window start (tiles tb .. tb+ntiles-1)
  int kend = a.Lk;
  if (a.mask_kind == kMaskCausal) kend = min(a.Lk, min(qb * bm + bm, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  int kbeg = 0;
  if (a.window > 0) kbeg = min(max(0, qb * bm + shift - a.window + 1), kend);
  const int tb = kbeg / BN;
  const int ntiles = max((kend + BN - 1) / BN - tb, 0);

  const bool wave_live = wi0 < a.Lq;
  const int w_last = min(wi0 + MF, a.Lq) - 1;
  int w_kend = a.Lk, w_kfull = a.Lk;
  if (a.mask_kind == kMaskCausal) {
    w_kend = min(a.Lk, w_last + shift + 1);
    w_kfull = min(a.Lk, wi0 + shift + 1);
  } else if (ADD || a.mask_kind == kMaskBool) {
    w_kfull = 0;
  }
  // with a window: keys below w_kskip are outside every row's window, keys
  // from w_klo on inside every row's (lower bound)
  int w_kskip = 0, w_klo = 0;
  if (a.window > 0) {
    w_kskip = wi0 + shift - a.window + 1;
    w_klo = w_last + shift - a.window + 1;
  }

  // Q fragment (B operand of S^T = K Q^T): row iq, k-elements kg*8.. of each KW chunk.
  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
  u32x4 qop[C::NQC];
#pragma unroll
  for (int c = 0; c < C::NQC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (iq < a.Lq) x = ld_global16(qp + c * C::KW + kg * 8);
    qop[c] = x ^ a.qsign;
  }

  if constexpr (C::DVP > DV) {
    for (int e = tid; e < BN * (C::DVP - DV); e += C::NT) {
      const int r = e / (C::DVP - DV), cc = DV + e % (C::DVP - DV);
      Vs[r * C::VST + cc] = 0;
    }
  }

  acc_t o[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) o[d] = acc_t{};
  float m = -INFINITY, l = 0.0f, sink2 = 0.0f;
  const bool has_sink = a.sinks != nullptr;
  if (has_sink) {
    sink2 = half_to_f32<E>(((const uint16_t*)a.sinks)[h]) * kLog2e;
    m = sink2;
  }

  const uint16_t* kp = (const uint16_t*)a.k + b * a.ks[0] + hkv * a.ks[1];
  const uint16_t* vp = (const uint16_t*)a.v + b * a.vs[0] + hkv * a.vs[1];
  const int64_t ksl = a.ks[2], vsl = a.vs[2];
  // additive mask: the lane's row (clamped for lanes past the last query row)
  const void* arow = nullptr;
  if constexpr (ADD)
    arow = (const uint16_t*)a.amask + b * a.ms[0] + h * a.ms[1] + (int64_t)min(iq, a.Lq - 1) * a.ms[2];
  // boolean mask: the lane's row of packed mask words (tile t covers words
  // t*BN/32 ..), fetched with the K/V tile one step ahead
  constexpr int MWT = BN / 32;
  static_assert(BN % 32 == 0, "tiles hold whole mask words");
  const bool bool_mask = a.mask_kind == kMaskBool;
  const uint32_t* mbrow = bool_mask ? a.mbits + (size_t)min(iq, a.Lq - 1) * a.mwords : nullptr;
  uint32_t mwn[MWT], mwc[MWT];
#pragma unroll
  for (int w = 0; w < MWT; ++w) mwn[w] = mwc[w] = 0u;

  u32x4 kr[C::KPT], vr[C::VPT];
  // additive mask: the lane's values for the next tile (mnx) and this one (mcu)
  constexpr int MG = ADD ? C::NSB * ACC / 4 : 1;
  u32x2 mnx[MG], mcu[MG];
  auto load_tile = [&](int k0) {
    if constexpr (ADD) {
      if (wave_live) {
#pragma unroll
        for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
          for (int g = 0; g < ACC / 4; ++g)
            mnx[nb * (ACC / 4) + g] = mask4_bits<E>(arow, k0 + nb * MF + acc_row<MF>(4 * g, kg), a.Lk);
      }
    }
    if (bool_mask) {
#pragma unroll
      for (int w = 0; w < MWT; ++w) {
        const int idx = k0 / 32 + w;
        mwn[w] = idx < a.mwords ? mbrow[idx] : 0u;
      }
    }
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int r = c / (D / 8), cc = c % (D / 8);
        const int key = k0 + r;
        kr[it] = key < a.Lk ? ld_global16(kp + key * ksl + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int r = c / (DV / 8), cc = c % (DV / 8);
        const int key = k0 + r;
        vr[it] = key < a.Lk ? ld_global16(vp + key * vsl + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int r = c / (D / 8), cc = c % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[r * C::KST + cc * 8]) = kr[it];
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int r = c / (DV / 8), cc = c % (DV / 8);
        *reinterpret_cast<u32x4*>(&Vs[r * C::VST + cc * 8]) = vr[it];
      }
    }
  };

  // transpose-read provider coordinates (see lds_read_tr16)
  const int tr_e = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int tr_dv = ((lane >> 4) * 16) % MF + 4 * tr_c;

  if (ntiles > 0) load_tile(tb * BN);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = (tb + t) * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
#pragma unroll
    for (int w = 0; w < MWT; ++w) mwc[w] = mwn[w];
    if constexpr (ADD) {
#pragma unroll
      for (int g = 0; g < MG; ++g) mcu[g] = mnx[g];
    }
    if (t + 1 < ntiles) load_tile(k0 + BN);
    if (!wave_live || k0 >= w_kend || k0 + BN <= w_kskip) continue;
    const bool full = k0 + BN <= w_kfull && k0 >= w_klo;

    // S^T = K Q^T
    acc_t s[C::NSB];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      acc_t acc = acc_t{};
#pragma unroll
      for (int c = 0; c < C::NQC; ++c) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(&Ks[(nb * MF + col) * C::KST + c * C::KW + kg * 8]);
        acc = mma16<E, MF>(kop, qop[c], acc);
      }
      s[nb] = acc;
    }

    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) mx = fmaxf(mx, s[nb][i]);
    } else if (ADD) {
      // base-2 scores with the mask added; keys past Lk carry -inf from the mask read
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) {
          s[nb][i] = iq < a.Lq ? fmaf(s[nb][i], a.c, mask_bits_value<E>(mcu[nb * (ACC / 4) + i / 4], i % 4))
                               : -INFINITY;
          mx = fmaxf(mx, s[nb][i]);
        }
    } else if (bool_mask) {
      // lane's keys: nb*MF + acc_row(i, 0) + 4 kg; packed bits are zero past Lk
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb) {
        const uint32_t wsh = iq < a.Lq ? (mwc[(nb * MF) / 32] >> (4 * kg)) : 0u;
#pragma unroll
        for (int i = 0; i < ACC; ++i) {
          s[nb][i] = keep_if_bit(s[nb][i], wsh, (nb * MF) % 32 + acc_row<MF>(i, 0));
          mx = fmaxf(mx, s[nb][i]);
        }
      }
    } else {
      // causal diagonal and window edge, or keys past Lk
      const int lim = a.mask_kind == kMaskCausal ? min(iq + shift, a.Lk - 1) : a.Lk - 1;
      const int lo = a.window > 0 ? iq + shift - a.window : -1;
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          const bool vis = (iq < a.Lq) & (key <= lim) & (key > lo);
          s[nb][i] = vis ? s[nb][i] : -INFINITY;
          mx = fmaxf(mx, s[nb][i]);
        }
    }
    // scores are in base 2 already with an additive mask, else scaled here
    const float sc = ADD ? 1.0f : a.c;
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * sc;
    softmax_rebase<C::NDB>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;

    uint32_t pk[C::NSB * ACC / 2];
    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; i += 2) {
        const float p0 = fast_exp2(fmaf(s[nb][i], sc, -mu));
        const float p1 = fast_exp2(fmaf(s[nb][i + 1], sc, -mu));
        lsum += p0 + p1;
        pk[(nb * ACC + i) / 2] = pack2<E>(p0, p1);
      }
    l += lsum;

    // O^T += V^T P^T
#pragma unroll
    for (int t8 = 0; t8 < C::NPV; ++t8) {
      const u32x4 pb = {pk[4 * t8], pk[4 * t8 + 1], pk[4 * t8 + 2], pk[4 * t8 + 3]};
      const int keyA = ((8 * t8) / ACC) * MF + acc_row<MF>((8 * t8) % ACC, kg);
      const int keyB = ((8 * t8 + 4) / ACC) * MF + acc_row<MF>((8 * t8 + 4) % ACC, kg);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const u32x2 ra = lds_read_tr16(&Vs[(keyA + tr_e) * C::VST + db * MF + tr_dv]);
        const u32x2 rb = lds_read_tr16(&Vs[(keyB + tr_e) * C::VST + db * MF + tr_dv]);
        const u32x4 va = {ra[0], ra[1], rb[0], rb[1]};
        o[db] = mma16<E, MF>(va, pb, o[db]);
      }
    }
  }

  if (!wave_live) return;
  float lt = row_sum<MF>(l);
  if (has_sink) lt += fast_exp2(sink2 - m);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (iq >= a.Lq) return;
  uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < ACC / 4; ++g4) {
      const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
      if (dv < DV) {
        const u32x2 st = {pack2<E>(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv),
                          pack2<E>(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv)};
        st_global8(op + dv, st);
      }
    }
}

// float32 inputs: the same walk on f32 MFMA (32x32x2 / 16x16x4), one k-element per lane.
template <int MF, int D, int DV, int BN, int NW>
struct PrefillCfgF32 {
  static constexpr int KWF = Mfma<MF>::KWF, ACC = Mfma<MF>::ACC, KG = Mfma<MF>::KG;
  static constexpr int DVP = (DV + MF - 1) / MF * MF;
  static constexpr int KST = D + 1;
  static constexpr int VST = DVP + MF;
  static constexpr int NQS = D / KWF;
  static constexpr int NSB = BN / MF;
  static constexpr int NDB = DVP / MF;
  static constexpr int NT = NW * 64;
  static constexpr int KCH = BN * D / 4, VCH = BN * DV / 4;
  static constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT;
  static constexpr int LDS_ELEMS = BN * KST + BN * VST;
  static_assert(D % KWF == 0 && BN % MF == 0, "shape");
};

// PAGED: K and V are paged caches ([blocks, Hkv, bs, D/Dv]); batch item b has
// lengths[b] keys (clamped to [0, max_blocks * bs]), key j in row j % bs of
// block table[b][j / bs] (clamped to [0, blocks - 1]); the causal mask and the
// window are aligned to that length (nuvec-core "tests/fast.rs",
// paged_attention_equals_contiguous_attention and its f32 cases).
template <int MF, int D, int DV, int BN, int NW, bool ADD, bool PAGED = false>
__global__ void __launch_bounds__(NW * 64) prefill_f32_kernel(FwdArgs a) {
  using C = PrefillCfgF32<MF, D, DV, BN, NW>;
  using acc_t = typename Mfma<MF>::acc_t;
  constexpr int ACC = C::ACC;
  __shared__ __attribute__((aligned(16))) float lds[C::LDS_ELEMS];
  float* Ks = lds;
  float* Vs = lds + BN * C::KST;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane % MF;
  const int kg = lane / MF;

  const int heads = a.Hq * a.B / a.head_blocks;
  const int wph = NW / heads;
  const int bm = wph * MF;
  int hb, qb;
  prefill_item((int)blockIdx.x, a.head_blocks, a.nqb, a.group / heads, hb, qb);
  const int groups_per_b = a.Hq / heads;
  const int b = hb / groups_per_b;
  const int h0 = (hb % groups_per_b) * heads;
  const int hkv = h0 / a.group;
  const int h = h0 + w / wph;
  const int wi0 = qb * bm + (w % wph) * MF;
  const int iq = wi0 + col;
  // the keys this batch item holds: all Lk, or the sequence's clamped length
  int Lk = a.Lk;
  if constexpr (PAGED) Lk = min(max(a.lengths[b], 0), a.max_blocks * a.bs);
  const int shift = Lk - a.Lq;

  // keys the workgroup needs: up to its last row's causal limit and, with a
  // sliding window, from its first row's window start (tiles tb .. tb+ntiles-1)
  int kend = Lk;
  if (a.mask_kind == kMaskCausal) kend = min(Lk, min(qb * bm + bm, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  int kbeg = 0;
  if (a.window > 0) kbeg = min(max(0, qb * bm + shift - a.window + 1), kend);
  const int tb = kbeg / BN;
  const int ntiles = max((kend + BN - 1) / BN - tb, 0);

  const bool wave_live = wi0 < a.Lq;
  const int w_last = min(wi0 + MF, a.Lq) - 1;
  int w_kend = Lk, w_kfull = Lk;
  if (a.mask_kind == kMaskCausal) {
    w_kend = min(Lk, w_last + shift + 1);
    w_kfull = min(Lk, wi0 + shift + 1);
  } else if (ADD || a.mask_kind == kMaskBool) {
    w_kfull = 0;
  }
  // with a window: keys below w_kskip are outside every row's window, keys
  // from w_klo on inside every row's (lower bound)
  int w_kskip = 0, w_klo = 0;
  if (a.window > 0) {
    w_kskip = wi0 + shift - a.window + 1;
    w_klo = w_last + shift - a.window + 1;
  }

  const float* qp = (const float*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
  float qop[C::NQS];
#pragma unroll
  for (int s = 0; s < C::NQS; ++s) {
    uint32_t x = 0u;
    if (iq < a.Lq) x = __float_as_uint(qp[s * C::KWF + kg]);
    qop[s] = __uint_as_float(x ^ a.qsign);
  }

  if constexpr (C::DVP > DV) {
    for (int e = tid; e < BN * (C::DVP - DV); e += C::NT) {
      const int r = e / (C::DVP - DV), cc = DV + e % (C::DVP - DV);
      Vs[r * C::VST + cc] = 0.0f;
    }
  }

  acc_t o[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) o[d] = acc_t{};
  float m = -INFINITY, l = 0.0f, sink2 = 0.0f;
  const bool has_sink = a.sinks != nullptr;
  if (has_sink) {
    sink2 = ((const float*)a.sinks)[h] * kLog2e;
    m = sink2;
  }

  const float* kp = (const float*)a.k + (PAGED ? 0 : b * a.ks[0] + hkv * a.ks[1]);
  const float* vp = (const float*)a.v + (PAGED ? 0 : b * a.vs[0] + hkv * a.vs[1]);
  const int64_t ksl = a.ks[2], vsl = a.vs[2];
  // paged: cache row of key `key` through the (clamped) block table
  const int32_t* trow = PAGED ? a.table + (size_t)b * a.max_blocks : nullptr;
  auto cache_row = [&](int key) -> int64_t {
    const int blk = min(max(trow[key / a.bs], 0), a.blocks - 1);
    return ((int64_t)blk * a.Hkv + hkv) * a.bs + key % a.bs;
  };
  const void* arow = nullptr;
  if constexpr (ADD)
    arow = (const float*)a.amask + b * a.ms[0] + h * a.ms[1] + (int64_t)min(iq, a.Lq - 1) * a.ms[2];
  const uint8_t* mrow = a.mask + (size_t)iq * a.Lk;

  u32x4 kr[C::KPT], vr[C::VPT];
  // additive mask: the lane's values for the next tile (mnx) and this one (mcu)
  constexpr int MG = ADD ? C::NSB * ACC / 4 : 1;
  f32x4 mnx[MG], mcu[MG];
  auto load_tile = [&](int k0) {
    if constexpr (ADD) {
      if (wave_live) {
#pragma unroll
        for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
          for (int g = 0; g < ACC / 4; ++g)
            mnx[nb * (ACC / 4) + g] =
                mask4_f32(arow, k0 + nb * MF + acc_row<MF>(4 * g, kg), a.Lk);
      }
    }
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int r = c / (D / 4), cc = c % (D / 4);
        const int key = k0 + r;
        // paged: keys before the workgroup's first visible key are not read (a
        // cache may hold anything there, e.g. blocks wholly before a window)
        const bool live = key < Lk && (!PAGED || key >= kbeg);
        const int64_t off = PAGED ? (live ? cache_row(key) * D : 0) : key * ksl;
        kr[it] = live ? ld_global16(kp + off + cc * 4) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int r = c / (DV / 4), cc = c % (DV / 4);
        const int key = k0 + r;
        const bool live = key < Lk && (!PAGED || key >= kbeg);
        const int64_t off = PAGED ? (live ? cache_row(key) * DV : 0) : key * vsl;
        vr[it] = live ? ld_global16(vp + off + cc * 4) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int r = c / (D / 4), cc = c % (D / 4);
        float* dst = &Ks[r * C::KST + cc * 4];   // odd row stride: scalar stores
        dst[0] = __uint_as_float(kr[it][0]);
        dst[1] = __uint_as_float(kr[it][1]);
        dst[2] = __uint_as_float(kr[it][2]);
        dst[3] = __uint_as_float(kr[it][3]);
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int r = c / (DV / 4), cc = c % (DV / 4);
        *reinterpret_cast<u32x4*>(&Vs[r * C::VST + cc * 4]) = vr[it];
      }
    }
  };

  if (ntiles > 0) load_tile(tb * BN);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = (tb + t) * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if constexpr (ADD) {
#pragma unroll
      for (int g = 0; g < MG; ++g) mcu[g] = mnx[g];
    }
    if (t + 1 < ntiles) load_tile(k0 + BN);
    if (!wave_live || k0 >= w_kend || k0 + BN <= w_kskip) continue;
    const bool full = k0 + BN <= w_kfull && k0 >= w_klo;

    acc_t s[C::NSB];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      acc_t acc = acc_t{};
#pragma unroll
      for (int st = 0; st < C::NQS; ++st)
        acc = mma_f32<MF>(Ks[(nb * MF + col) * C::KST + st * C::KWF + kg], qop[st], acc);
      s[nb] = acc;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        if (ADD) {
          // base-2 scores with the mask added; keys past Lk carry -inf from the mask read
          s[nb][i] = iq < a.Lq ? fmaf(s[nb][i], a.c, mcu[nb * (ACC / 4) + i / 4][i % 4]) : -INFINITY;
        } else if (!full) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          bool vis = key < Lk && iq < a.Lq;
          if (a.mask_kind == kMaskCausal)
            vis = vis && key <= iq + shift && (a.window <= 0 || key > iq + shift - a.window);
          else if (a.mask_kind == kMaskBool) vis = vis && mrow[key] != 0;
          if (!vis) s[nb][i] = -INFINITY;
        }
        mx = fmaxf(mx, s[nb][i]);
      }
    const float sc = ADD ? 1.0f : a.c;
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * sc;
    softmax_rebase<C::NDB>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;

    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        const float p = fast_exp2(fmaf(s[nb][i], sc, -mu));
        s[nb][i] = p;
        lsum += p;
      }
    l += lsum;

    // O^T += V^T P^T, one key per lane k-group and instruction
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        const int key = nb * MF + acc_row<MF>(i, kg);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          o[db] = mma_f32<MF>(Vs[key * C::VST + db * MF + col], s[nb][i], o[db]);
      }
  }

  if (!wave_live) return;
  float lt = row_sum<MF>(l);
  if (has_sink) lt += fast_exp2(sink2 - m);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (iq >= a.Lq) return;
  float* op = (float*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < ACC / 4; ++g4) {
      const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
      if (dv < DV) {
        const f32x4 st = {o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv,
                          o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv};
        *reinterpret_cast<f32x4*>(op + dv) = st;
      }
    }
}

}  // namespace sdpa

namespace sdpa {

// float32, small calls: the NW wavefronts of a workgroup share one 16-row
// query block of one head and split its key tiles among themselves (wave w
// takes tiles w, w + NW, ...), each staging its own tiles in a private LDS
// region, so the walk needs no workgroup barrier and the longest row block's
// keys are walked NW ways in parallel. At the end the waves' running maxima,
// sums and unnormalised outputs meet in LDS and are merged with the same
// log-sum-exp combine as the decode splits (nuvec-core "tests/attention_plan.rs":
// a split key axis whose partial results a second step combines), exactly, up
// to rounding. Masks, windows, sinks, strided q/k/v and paged caches (PAGED) as
// in prefill_f32_kernel; no additive mask.
template <int D, int DV, int BN, int NW>
struct PrefillCfgF32Split {
  static constexpr int MF = 16;
  static constexpr int KWF = Mfma<MF>::KWF, ACC = Mfma<MF>::ACC, KG = Mfma<MF>::KG;
  static constexpr int DVP = (DV + MF - 1) / MF * MF;
  static constexpr int KST = D + 1;
  static constexpr int VST = DVP + MF;
  static constexpr int NQS = D / KWF;
  static constexpr int NSB = BN / MF;
  static constexpr int NDB = DVP / MF;
  static constexpr int KCH = BN * D / 4, VCH = BN * DV / 4;  // 16-byte chunks per tile
  static constexpr int KPT = (KCH + 63) / 64, VPT = (VCH + 63) / 64;
  static constexpr int WAVE_ELEMS = BN * KST + BN * VST;      // one wave's tile region
  static constexpr int MERGE_ELEMS = MF * DVP + 2 * MF;       // one wave's partial rows
  static constexpr int REGION = WAVE_ELEMS > MERGE_ELEMS ? WAVE_ELEMS : MERGE_ELEMS;
  static_assert(D % KWF == 0 && BN % MF == 0, "shape");
};

template <int D, int DV, int BN, int NW, bool PAGED>
__global__ void __launch_bounds__(NW * 64) prefill_f32_split_kernel(FwdArgs a) {
  using C = PrefillCfgF32Split<D, DV, BN, NW>;
  constexpr int MF = C::MF, ACC = C::ACC;
  using acc_t = typename Mfma<MF>::acc_t;
  __shared__ __attribute__((aligned(16))) float lds[NW * C::REGION];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane % MF;
  const int kg = lane / MF;
  float* Ks = lds + w * C::REGION;
  float* Vs = Ks + BN * C::KST;

  // workgroup n: (batch, head) n / nqb, query block nqb - 1 - n % nqb (long blocks first)
  const int n = blockIdx.x;
  const int bh = n / a.nqb;
  const int qb = a.nqb - 1 - n % a.nqb;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hkv = h / a.group;
  const int i0 = qb * MF;
  const int iq = i0 + col;
  // the keys this batch item holds: all Lk, or the sequence's clamped length
  int Lk = a.Lk;
  if constexpr (PAGED) Lk = min(max(a.lengths[b], 0), a.max_blocks * a.bs);
  const int shift = Lk - a.Lq;

  int kend = Lk;
  if (a.mask_kind == kMaskCausal) kend = min(Lk, min(i0 + MF, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  int kbeg = 0;
  if (a.window > 0) kbeg = min(max(0, i0 + shift - a.window + 1), kend);
  const int tb = kbeg / BN;
  const int ntiles = max((kend + BN - 1) / BN - tb, 0);
  // keys every row sees, [w_klo, w_kfull)
  int w_kfull = a.mask_kind == kMaskBool ? 0 : Lk;
  if (a.mask_kind == kMaskCausal) w_kfull = min(Lk, i0 + shift + 1);
  int w_klo = 0;
  if (a.window > 0) w_klo = min(i0 + MF, a.Lq) - 1 + shift - a.window + 1;

  const float* qp = (const float*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
  float qop[C::NQS];
#pragma unroll
  for (int st = 0; st < C::NQS; ++st) {
    uint32_t x = 0u;
    if (iq < a.Lq) x = __float_as_uint(qp[st * C::KWF + kg]);
    qop[st] = __uint_as_float(x ^ a.qsign);
  }
  if constexpr (C::DVP > DV) {
    for (int e = lane; e < BN * (C::DVP - DV); e += 64) {
      const int r = e / (C::DVP - DV), cc = DV + e % (C::DVP - DV);
      Vs[r * C::VST + cc] = 0.0f;
    }
  }

  acc_t o[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) o[d] = acc_t{};
  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? ((const float*)a.sinks)[h] * kLog2e : -INFINITY;
  float m = sink2, l = 0.0f;

  // strided: this (batch, kv head)'s rows; paged: the cache base (rows through the table)
  const float* kp = (const float*)a.k + (PAGED ? 0 : b * a.ks[0] + hkv * a.ks[1]);
  const float* vp = (const float*)a.v + (PAGED ? 0 : b * a.vs[0] + hkv * a.vs[1]);
  const uint8_t* mrow = a.mask + (size_t)min(iq, a.Lq - 1) * a.Lk;
  const int32_t* trow = PAGED ? a.table + (size_t)b * a.max_blocks : nullptr;
  auto cache_row = [&](int key) -> int64_t {
    const int blk = min(max(trow[key / a.bs], 0), a.blocks - 1);
    return ((int64_t)blk * a.Hkv + hkv) * a.bs + key % a.bs;
  };

  u32x4 kr[C::KPT], vr[C::VPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = lane + it * 64;
      if (C::KCH % 64 == 0 || c < C::KCH) {
        const int r = c / (D / 4), cc = c % (D / 4);
        const int key = k0 + r;
        // paged: keys before the workgroup's first visible key are not read
        const bool live = key < Lk && (!PAGED || key >= kbeg);
        const int64_t off = PAGED ? (live ? cache_row(key) * D : 0) : key * a.ks[2];
        kr[it] = live ? ld_global16(kp + off + cc * 4) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = lane + it * 64;
      if (C::VCH % 64 == 0 || c < C::VCH) {
        const int r = c / (DV / 4), cc = c % (DV / 4);
        const int key = k0 + r;
        const bool live = key < Lk && (!PAGED || key >= kbeg);
        const int64_t off = PAGED ? (live ? cache_row(key) * DV : 0) : key * a.vs[2];
        vr[it] = live ? ld_global16(vp + off + cc * 4) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // the wave's own region: its LDS writes and reads stay in order within the wave
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = lane + it * 64;
      if (C::KCH % 64 == 0 || c < C::KCH) {
        const int r = c / (D / 4), cc = c % (D / 4);
        float* dst = &Ks[r * C::KST + cc * 4];   // odd row stride: scalar stores
        dst[0] = __uint_as_float(kr[it][0]);
        dst[1] = __uint_as_float(kr[it][1]);
        dst[2] = __uint_as_float(kr[it][2]);
        dst[3] = __uint_as_float(kr[it][3]);
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = lane + it * 64;
      if (C::VCH % 64 == 0 || c < C::VCH) {
        const int r = c / (DV / 4), cc = c % (DV / 4);
        *reinterpret_cast<u32x4*>(&Vs[r * C::VST + cc * 4]) = vr[it];
      }
    }
  };

  int t = w;
  if (t < ntiles) load_tile((tb + t) * BN);
  for (; t < ntiles; t += NW) {
    const int k0 = (tb + t) * BN;
    __builtin_amdgcn_wave_barrier();
    store_tile();
    __builtin_amdgcn_wave_barrier();
    if (t + NW < ntiles) load_tile(k0 + NW * BN);
    const bool full = k0 + BN <= w_kfull && k0 >= w_klo;

    acc_t s[C::NSB];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      acc_t acc = acc_t{};
#pragma unroll
      for (int st = 0; st < C::NQS; ++st)
        acc = mma_f32<MF>(Ks[(nb * MF + col) * C::KST + st * C::KWF + kg], qop[st], acc);
      s[nb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        if (!full) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          bool vis = key < Lk && iq < a.Lq;
          if (a.mask_kind == kMaskCausal)
            vis = vis && key <= iq + shift && (a.window <= 0 || key > iq + shift - a.window);
          else if (a.mask_kind == kMaskBool) vis = vis && mrow[key] != 0;
          if (!vis) s[nb][i] = -INFINITY;
        }
        mx = fmaxf(mx, s[nb][i]);
      }
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * a.c;
    softmax_rebase<C::NDB>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;
    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        const float p = fast_exp2(fmaf(s[nb][i], a.c, -mu));
        s[nb][i] = p;
        lsum += p;
      }
    l += lsum;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        const int key = nb * MF + acc_row<MF>(i, kg);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          o[db] = mma_f32<MF>(Vs[key * C::VST + db * MF + col], s[nb][i], o[db]);
      }
  }

  // merge: each wave leaves its rows' reference maximum, sum and unnormalised
  // output in its region; wave w then combines the value-column blocks
  // db = w, w + NW, ... of every row
  const float lt = row_sum<MF>(l);
  __syncthreads();
  float* part = lds + w * C::REGION;
  if (kg == 0) {
    part[MF * C::DVP + col] = m;
    part[MF * C::DVP + MF + col] = lt;
  }
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
    *reinterpret_cast<f32x4*>(&part[col * C::DVP + db * MF + kg * 4]) = o[db];
  __syncthreads();
  float mw[NW], M = sink2;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    mw[u] = lds[u * C::REGION + MF * C::DVP + col];
    M = fmaxf(M, mw[u]);
  }
  float fw[NW], L = 0.0f;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    fw[u] = mw[u] == -INFINITY ? 0.0f : fast_exp2(mw[u] - M);
    L += lds[u * C::REGION + MF * C::DVP + MF + col] * fw[u];
  }
  if (has_sink && M != -INFINITY) L += fast_exp2(sink2 - M);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (iq >= a.Lq) return;
  float* op = (float*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV;
  for (int db = w; db < C::NDB; db += NW) {
    const int dv = db * MF + kg * 4;
    if (dv >= DV) continue;
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < NW; ++u) x += *reinterpret_cast<const f32x4*>(&lds[u * C::REGION + col * C::DVP + dv]) * fw[u];
    *reinterpret_cast<f32x4*>(op + dv) = x * inv;
  }
}

}  // namespace sdpa
