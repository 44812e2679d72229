// Decode: split-key two-pass attention for few query rows per key/value head.
//
// First pass (decode_split_kernel): one workgroup of NW wavefronts per (batch,
// kv head, key split). All Hq/Hkv x Lq query rows that read this kv head are
// packed into one MFMA tile, so every K/V byte is fetched once for the whole
// group. The workgroup streams its keys in tiles of BN: each tile's K and V
// rows are loaded by all threads with 16-byte streaming loads (the next two
// tiles' loads are in flight while the current tile is computed; each
// workgroup reads one contiguous stretch of K and of V) and staged once in LDS. Every
// wavefront forms the scores and softmax weights of the tile (S^T = K Q^T on
// MFMA; this redundant work is small), then accumulates its own share of the
// value columns (O^T += V^T P^T, V^T via LDS transpose reads). The workgroup
// leaves, per query row, its maximum m (base 2), its sum of weights l and its
// unnormalised output in the scratch buffer: per row a 16-byte {m, l} slot in
// a first region, and Dv floats in a second.
//
// Second pass (decode_reduce_kernel): per query row, the log-sum-exp combine
// of the splits with the sink logit as one more term of the denominator, one
// division and the single rounding to the output type. The two passes are the
// split/reduce pair named by nuvec-core "tests/attention_plan.rs" (first-pass
// dispatches over key partitions, then a second pass).
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int MF, int D, int DV, int NW>
struct DecodeCfg {
  static constexpr int KW = Mfma<MF>::KW, ACC = Mfma<MF>::ACC, KG = Mfma<MF>::KG;
  static constexpr int BN = kDecodeBN;
  static constexpr int DVP = (DV + MF - 1) / MF * MF;
  static constexpr int KST = D + 8;        // LDS row strides (elements)
  static constexpr int VST = DVP + 16;
  static constexpr int NQC = D / KW;
  static constexpr int NSB = BN / MF;
  static constexpr int NPV = BN / KW;
  static constexpr int NDB = DVP / MF;            // value-column blocks in all
  static constexpr int NDBW = (NDB + NW - 1) / NW; // blocks per wavefront (at most)
  static constexpr int NT = NW * 64;
  static constexpr int KCH = BN * D / 8, VCH = BN * DV / 8;
  static constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT;
  static constexpr int LDS_ELEMS = BN * KST + BN * VST;
  static_assert(D % KW == 0, "head size must be a whole number of MFMA k-steps");
};

// PAGED: K and V are paged caches ([blocks, Hkv, bs, D]); sequence b has
// lengths[b] keys (clamped to [0, max_blocks * bs]), key j in row j % bs of
// block table[b][j / bs] (clamped to [0, blocks - 1]). The split's table
// entries are staged in LDS once, so each key row's address needs no further
// global read (nuvec-core "tests/fast.rs", paged_attention_equals_contiguous_
// attention and paged_attention_clamps_hostile_tables_and_lengths).
template <class E, int MF, int D, int DV, int NW, bool PAGED = false>
__global__ void __launch_bounds__(NW * 64) decode_split_kernel(FwdArgs a) {
  using C = DecodeCfg<MF, D, DV, NW>;
  using acc_t = typename Mfma<MF>::acc_t;
  constexpr int ACC = C::ACC;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* Ks = lds;
  uint16_t* Vs = lds + BN * C::KST;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane % MF;
  const int kg = lane / MF;

  // Dispatch order: splits 0 .. nsplit-2 of each (kv head, batch item) pair,
  // pair after pair, then the last split of every pair. The last split is the
  // shortest, so when the grid overflows the compute units by a few
  // workgroups (260 for 256 at 8193 keys and four kv heads) the overflow is
  // made of short splits rather than full ones (12.7 -> 11.8 us there).
  const int64_t lin = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t per = a.nsplit > 1 ? a.nsplit - 1 : 1;   // splits before the last one
  const int64_t nbulk = (int64_t)a.Hkv * a.B * (a.nsplit - 1);
  const int64_t pair = lin < nbulk ? lin / per : lin - nbulk;
  const int split = lin < nbulk ? (int)(lin % per) : a.nsplit - 1;
  const int hkv = (int)(pair % a.Hkv);
  const int b = (int)(pair / a.Hkv);
  // the keys this batch item holds: all Lk, or the sequence's clamped length
  int Lk = a.Lk, koff = a.koff;
  if constexpr (PAGED) {
    Lk = min(max(a.lengths[b], 0), a.max_blocks * a.bs);
    koff = a.window > 0 ? max(0, Lk - a.Lq - a.window + 1) : 0;
  }
  // splits cover the keys the rows read: with a sliding window, from koff
  const int ks = koff + split * a.kps;
  const int ke = min(ks + a.kps, Lk);
  const int ntiles = ks < ke ? (ke - ks + BN - 1) / BN : 0;
  // paged: clamped block ids of this split's keys (at most kps + 1 <= 1025)
  __shared__ int32_t ptab[PAGED ? 1025 : 1];
  const int e0 = PAGED ? ks / max(a.bs, 1) : 0;
  if constexpr (PAGED) {
    const int ne = ntiles > 0 ? (ke - 1) / a.bs - e0 + 1 : 0;
    for (int i = threadIdx.x; i < ne; i += NW * 64)
      ptab[i] = min(max(a.table[(size_t)b * a.max_blocks + e0 + i], 0), a.blocks - 1);
    __syncthreads();
  }

  // packed query rows: row r -> head hkv*group + r / Lq, position r % Lq
  const int r = col;
  const bool row_ok = r < a.rows;
  const int h = hkv * a.group + (row_ok ? r / a.Lq : 0);
  const int iq = row_ok ? r % a.Lq : 0;
  const int shift = Lk - a.Lq;

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
  u32x4 qop[C::NQC];
#pragma unroll
  for (int c = 0; c < C::NQC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = ld_global16(qp + c * C::KW + kg * 8);
    qop[c] = x ^ a.qsign;
  }

  if constexpr (C::DVP > DV) {
    for (int e = tid; e < BN * (C::DVP - DV); e += C::NT) {
      const int rr = e / (C::DVP - DV), cc = DV + e % (C::DVP - DV);
      Vs[rr * C::VST + cc] = 0;
    }
  }

  acc_t o[C::NDBW];
#pragma unroll
  for (int d = 0; d < C::NDBW; ++d) o[d] = acc_t{};
  float m = -INFINITY, l = 0.0f;

  // strided: this (batch, kv head)'s rows; paged: the cache base (rows through the table)
  const uint16_t* kp = (const uint16_t*)a.k + (PAGED ? 0 : b * a.ks[0] + hkv * a.ks[1]);
  const uint16_t* vp = (const uint16_t*)a.v + (PAGED ? 0 : b * a.vs[0] + hkv * a.vs[1]);
  const uint8_t* mrow = a.mask + (size_t)iq * a.Lk;
  const bool causal_cut = a.mask_kind == kMaskCausal && a.Lq > 1;
  // additive mask: the lane's row (values in the element type, added in base 2)
  const bool additive = a.mask_kind == kMaskAdditive;
  const uint16_t* arow = additive ? (const uint16_t*)a.amask + b * a.ms[0] + h * a.ms[1] + (int64_t)iq * a.ms[2]
                                  : nullptr;
  const float sc = additive ? 1.0f : a.c;

  // Two register tiles (A and B) cycle so that two tiles of K/V loads are in
  // flight while the LDS copy of a third is being computed.
  u32x4 kra[C::KPT], vra[C::VPT], krb[C::KPT], vrb[C::VPT];
  // element offsets of key `key`'s K and V rows: strided, or through the block table
  auto k_off = [&](int key) -> int64_t {
    if constexpr (PAGED)
      return (((int64_t)ptab[key / a.bs - e0] * a.Hkv + hkv) * a.bs + key % a.bs) * D;
    else
      return key * a.ks[2];
  };
  auto v_off = [&](int key) -> int64_t {
    if constexpr (PAGED)
      return (((int64_t)ptab[key / a.bs - e0] * a.Hkv + hkv) * a.bs + key % a.bs) * DV;
    else
      return key * a.vs[2];
  };
  auto load_tile = [&](int k0, u32x4* kr, u32x4* vr) {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int rr = c / (D / 8), cc = c % (D / 8);
        const int key = min(k0 + rr, ke - 1);  // rows past the split's end re-read its last key (weight 0)
        kr[it] = ld_global16_nt(kp + k_off(key) + cc * 8);
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int rr = c / (DV / 8), cc = c % (DV / 8);
        const int key = min(k0 + rr, ke - 1);
        vr[it] = ld_global16_nt(vp + v_off(key) + cc * 8);
      }
    }
  };
  auto store_tile = [&](const u32x4* kr, const u32x4* vr) {
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::KCH % C::NT == 0 || c < C::KCH) {
        const int rr = c / (D / 8), cc = c % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[rr * C::KST + cc * 8]) = kr[it];
      }
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = tid + it * C::NT;
      if (C::VCH % C::NT == 0 || c < C::VCH) {
        const int rr = c / (DV / 8), cc = c % (DV / 8);
        *reinterpret_cast<u32x4*>(&Vs[rr * C::VST + cc * 8]) = vr[it];
      }
    }
  };

  const int tr_e = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int tr_dv = ((lane >> 4) * 16) % MF + 4 * tr_c;

  auto compute = [&](int k0) {
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

    const bool full = k0 + BN <= ke && a.mask_kind != kMaskBool && !additive && !causal_cut;
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        if (!full) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          bool vis = key < ke && row_ok;
          if (additive) {
            // base-2 score with the mask added
            float add = -INFINITY;
            if (vis) add = half_to_f32<E>(arow[key]) * kLog2e;
            s[nb][i] = vis ? fmaf(s[nb][i], a.c, add) : -INFINITY;
          } else {
            if (causal_cut) vis = vis && key <= iq + shift && (a.window <= 0 || key > iq + shift - a.window);
            else if (a.mask_kind == kMaskBool) vis = vis && mrow[key] != 0;
            if (!vis) s[nb][i] = -INFINITY;
          }
        }
        mx = fmaxf(mx, s[nb][i]);
      }
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * sc;
    softmax_rebase<C::NDBW>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;

    // weights rounded to 16 bits for the MFMA; the running sum adds the same
    // rounded weights, so numerator and denominator agree
    uint32_t pk[C::NSB * ACC / 2];
    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; i += 2) {
        const float p0 = fast_exp2(fmaf(s[nb][i], sc, -mu));
        const float p1 = fast_exp2(fmaf(s[nb][i + 1], sc, -mu));
        pk[(nb * ACC + i) / 2] = pack2<E>(p0, p1);
        lsum = pair_sum<E>(pk[(nb * ACC + i) / 2], lsum);
      }
    l += lsum;

#pragma unroll
    for (int t8 = 0; t8 < C::NPV; ++t8) {
      const u32x4 pb = {pk[4 * t8], pk[4 * t8 + 1], pk[4 * t8 + 2], pk[4 * t8 + 3]};
      const int keyA = ((8 * t8) / ACC) * MF + acc_row<MF>((8 * t8) % ACC, kg);
      const int keyB = ((8 * t8 + 4) / ACC) * MF + acc_row<MF>((8 * t8 + 4) % ACC, kg);
#pragma unroll
      for (int j = 0; j < C::NDBW; ++j) {
        const int db = w + NW * j;
        if (C::NDB % NW == 0 || db < C::NDB) {
          const u32x2 ra = lds_read_tr16(&Vs[(keyA + tr_e) * C::VST + db * MF + tr_dv]);
          const u32x2 rb = lds_read_tr16(&Vs[(keyB + tr_e) * C::VST + db * MF + tr_dv]);
          const u32x4 va = {ra[0], ra[1], rb[0], rb[1]};
          o[j] = mma16<E, MF>(va, pb, o[j]);
        }
      }
    }
  };

  // Every tile load is issued whatever the tile count (rows past the split's
  // end re-read its last key), so the loads in flight come in the same order
  // on every path: before a tile's registers go to LDS, exactly the other
  // tile's loads may still be outstanding, and a counted wait leaves them in
  // flight. Plain barriers: the fence of __syncthreads would drain them. The
  // walk is unrolled by four tiles because the compiler's own wait at the
  // loop's head still drains everything.
  constexpr int LPT = C::KPT + C::VPT;  // loads per tile and thread
  auto wait_tile = [&](bool other_in_flight) {
    if (other_in_flight) {
      __builtin_amdgcn_s_waitcnt((LPT & 15) | ((LPT >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    }
  };
  // one step: tile u's registers to LDS, tile u+2's loads into them, tile u computed
  auto step = [&](int u, u32x4* kr, u32x4* vr) {
    wait_tile(true);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    store_tile(kr, vr);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_tile(ks + (u + 2) * BN, kr, vr);
    compute(ks + u * BN);
  };
  if (ntiles > 0) {
    load_tile(ks, kra, vra);
    load_tile(ks + BN, krb, vrb);
    for (int t = 0; t < ntiles; t += 4) {
      step(t, kra, vra);
      if (t + 1 >= ntiles) break;
      step(t + 1, krb, vrb);
      if (t + 2 >= ntiles) break;
      step(t + 2, kra, vra);
      if (t + 3 >= ntiles) break;
      step(t + 3, krb, vrb);
    }
    wait_tile(false);  // the loads issued past the last tile
  }

  const float lt = row_sum<MF>(l);
  if (!row_ok) return;
  const size_t prow = ((size_t)(b * a.Hkv + hkv) * a.nsplit + split) * a.rows + r;
  const size_t total_rows = (size_t)a.B * a.Hkv * a.nsplit * a.rows;
  float* pml = a.part + prow * 4;
  float* po = a.part + total_rows * 4 + prow * DV;
  if (w == 0 && kg == 0) {
    pml[0] = m;
    pml[1] = lt;
  }
#pragma unroll
  for (int j = 0; j < C::NDBW; ++j) {
    const int db = w + NW * j;
#pragma unroll
    for (int g4 = 0; g4 < ACC / 4; ++g4) {
      const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
      if ((C::NDB % NW == 0 || db < C::NDB) && dv < DV) {
        const f32x4 st = {o[j][g4 * 4 + 0], o[j][g4 * 4 + 1], o[j][g4 * 4 + 2], o[j][g4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(po + dv) = st;
      }
    }
  }
}

// One 256-thread workgroup per (query row and CS-column slice, kv head, batch
// item). Pass 1 finds
// the largest split maximum (with the sink). Pass 2 walks the splits in chunks
// of 256: each thread turns one split's maximum into its weight in LDS and adds
// that split's share of the sum; then SG groups of threads, each lane owning
// four value columns, add the weighted partial outputs of every SG-th split
// (independent loads, many in flight). The groups' sums meet in LDS.
template <class E, int DV>
__global__ void __launch_bounds__(256) decode_reduce_kernel(FwdArgs a) {
  constexpr int CS = reduce_cols(DV);  // value columns per workgroup
  constexpr int NCG = CS / 4;        // four-column groups
  constexpr int SG = 256 / NCG;      // split lanes
  static_assert(DV % CS == 0, "value columns split into whole slices");
  __shared__ float fw[256];
  __shared__ float red[4];
  __shared__ f32x4 accs[SG][NCG];
  const int r = blockIdx.x / (DV / CS), hkv = blockIdx.y, b = blockIdx.z;
  const int c0 = (blockIdx.x % (DV / CS)) * CS;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int h = hkv * a.group + r / a.Lq;
  const int iq = r % a.Lq;
  const size_t pair = (size_t)(b * a.Hkv + hkv);
  const size_t total_rows = (size_t)a.B * a.Hkv * a.nsplit * a.rows;
  const size_t row0 = pair * a.nsplit * a.rows + r;        // split sp's row: row0 + sp * rows
  const float* pml = a.part + row0 * 4;
  const float* po = a.part + total_rows * 4 + row0 * DV + c0;
  const size_t ml_step = (size_t)a.rows * 4, o_step = (size_t)a.rows * DV;

  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? half_to_f32<E>(((const uint16_t*)a.sinks)[h]) * kLog2e : -INFINITY;
  float M = -INFINITY;
  for (int sp = t; sp < a.nsplit; sp += 256) M = fmaxf(M, pml[sp * ml_step]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), sink2);

  const int cg = t % NCG, sg = t / NCG;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float lpart = 0.0f;
  if (M != -INFINITY) {
    for (int base = 0; base < a.nsplit; base += 256) {
      const int n = min(256, a.nsplit - base);
      __syncthreads();
      if (t < n) {
        const float ms = pml[(base + t) * ml_step];
        const float f = ms == -INFINITY ? 0.0f : fast_exp2(ms - M);  // empty splits hold zeros
        fw[t] = f;
        lpart += pml[(base + t) * ml_step + 1] * f;
      }
      __syncthreads();
      if (sg < SG) {
#pragma unroll 8
        for (int j = sg; j < n; j += SG)
          acc += *reinterpret_cast<const f32x4*>(po + (base + j) * o_step + cg * 4) * fw[j];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lpart += __shfl_xor(lpart, off);
  if (lane == 0) red[wv] = lpart;
  if (sg < SG) accs[sg][cg] = acc;
  __syncthreads();
  if (t >= NCG) return;
  float L = red[0] + red[1] + red[2] + red[3];
  if (has_sink && M != -INFINITY) L += fast_exp2(sink2 - M);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  f32x4 x = accs[0][t];
#pragma unroll
  for (int g = 1; g < SG; ++g) x += accs[g][t];
  x *= inv;
  uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV + c0;
  const u32x2 st = {pack2<E>(x[0], x[1]), pack2<E>(x[2], x[3])};
  st_global8(op + t * 4, st);
}

}  // namespace sdpa
