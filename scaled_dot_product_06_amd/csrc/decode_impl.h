// Decode: split-key two-pass attention for few query rows per key/value head.
//
// First pass (decode_split_kernel): one wavefront per (batch, kv head, key
// split). The wavefront packs all Hq/Hkv x Lq query rows that read this kv head
// into one MFMA tile, so each K/V byte is fetched once for the whole group.
// K fragments go straight from global memory into MFMA operands (16-byte
// loads); each 32-key V tile passes through a wavefront-private LDS buffer so
// that transpose reads can form the V^T operand. The wavefront leaves, per
// query row, its running maximum m (base 2), its sum of weights l and its
// unnormalised output in the scratch buffer (per row: a 16-byte {m, l}
// slot, then Dv floats in a second region).
//
// Second pass (decode_reduce_kernel): per query row, the log-sum-exp combine
// of the splits, plus the sink logit as one more term of the denominator, one
// division, and the single rounding to the output type. The two passes are
// the split/reduce pair named by nuvec-core "tests/attention_plan.rs"
// (first-pass dispatches over key partitions, then a second pass).
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int MF, int D, int DV>
struct DecodeCfg {
  static constexpr int KW = Mfma<MF>::KW, ACC = Mfma<MF>::ACC, KG = Mfma<MF>::KG;
  static constexpr int BN = kDecodeBN;
  static constexpr int DVP = (DV + MF - 1) / MF * MF;
  static constexpr int VST = DVP + 16;
  static constexpr int NQC = D / KW;
  static constexpr int NSB = BN / MF;
  static constexpr int NPV = BN / KW;
  static constexpr int NDB = DVP / MF;
  static constexpr int VCH = BN * DV / 8;
  static constexpr int VPT = (VCH + 63) / 64;
  static_assert(D % KW == 0, "head size must be a whole number of MFMA k-steps");
};

template <class E, int MF, int D, int DV, int NW>
__global__ void __launch_bounds__(NW * 64) decode_split_kernel(FwdArgs a) {
  using C = DecodeCfg<MF, D, DV>;
  using acc_t = typename Mfma<MF>::acc_t;
  constexpr int ACC = C::ACC;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint16_t lds[NW * BN * C::VST];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = lane % MF;
  const int kg = lane / MF;
  uint16_t* Vs = lds + w * BN * C::VST;

  const int split = (int)blockIdx.x * NW + w;
  const int hkv = blockIdx.y;
  const int b = blockIdx.z;
  if (split >= a.nsplit) return;
  const int ks = split * a.kps;
  const int ke = min(ks + a.kps, a.Lk);

  // packed query rows: row r -> head hkv*group + r / Lq, position r % Lq
  const int r = col;
  const bool row_ok = r < a.rows;
  const int h = hkv * a.group + (row_ok ? r / a.Lq : 0);
  const int iq = row_ok ? r % a.Lq : 0;
  const int shift = a.Lk - a.Lq;

  const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(b * a.Hq + h) * a.Lq + iq) * D;
  u32x4 qop[C::NQC];
#pragma unroll
  for (int c = 0; c < C::NQC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = ld_global16(qp + c * C::KW + kg * 8);
    qop[c] = x ^ a.qsign;
  }

  if constexpr (C::DVP > DV) {
    for (int e = lane; e < BN * (C::DVP - DV); e += 64) {
      const int rr = e / (C::DVP - DV), cc = DV + e % (C::DVP - DV);
      Vs[rr * C::VST + cc] = 0;
    }
  }

  acc_t o[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) o[d] = acc_t{};
  float m = -INFINITY, l = 0.0f;

  const uint16_t* kp = (const uint16_t*)a.k + (size_t)(b * a.Hkv + hkv) * (size_t)a.Lk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)(b * a.Hkv + hkv) * (size_t)a.Lk * DV;
  const uint8_t* mrow = a.mask + (size_t)iq * a.Lk;
  const bool causal_cut = a.mask_kind == kMaskCausal && a.Lq > 1;

  const int tr_e = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int tr_dv = ((lane >> 4) * 16) % MF + 4 * tr_c;

  for (int k0 = ks; k0 < ke; k0 += BN) {
    u32x4 kop[C::NSB][C::NQC];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      const int key = k0 + nb * MF + col;
#pragma unroll
      for (int c = 0; c < C::NQC; ++c)
        kop[nb][c] = key < ke ? ld_global16(kp + (size_t)key * D + c * C::KW + kg * 8)
                              : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 vr[C::VPT];
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = lane + it * 64;
      if (C::VCH % 64 == 0 || c < C::VCH) {
        const int rr = c / (DV / 8), cc = c % (DV / 8);
        const int key = k0 + rr;
        vr[it] = key < ke ? ld_global16(vp + (size_t)key * DV + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }

    acc_t s[C::NSB];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      acc_t acc = acc_t{};
#pragma unroll
      for (int c = 0; c < C::NQC; ++c) acc = mma16<E, MF>(kop[nb][c], qop[c], acc);
      s[nb] = acc;
    }

    const bool full = k0 + BN <= ke && a.mask_kind != kMaskBool && !causal_cut;
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; ++i) {
        if (!full) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          bool vis = key < ke && row_ok;
          if (causal_cut) vis = vis && key <= iq + shift;
          else if (a.mask_kind == kMaskBool) vis = vis && mrow[key] != 0;
          if (!vis) s[nb][i] = -INFINITY;
        }
        mx = fmaxf(mx, s[nb][i]);
      }
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * a.c;
    softmax_rebase<C::NDB>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;

    uint32_t pk[C::NSB * ACC / 2];
    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; i += 2) {
        const float p0 = fast_exp2(fmaf(s[nb][i], a.c, -mu));
        const float p1 = fast_exp2(fmaf(s[nb][i + 1], a.c, -mu));
        lsum += p0 + p1;
        pk[(nb * ACC + i) / 2] = pack2<E>(p0, p1);
      }
    l += lsum;

    // V tile into this wavefront's LDS buffer, then O^T += V^T P^T
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int c = lane + it * 64;
      if (C::VCH % 64 == 0 || c < C::VCH) {
        const int rr = c / (DV / 8), cc = c % (DV / 8);
        *reinterpret_cast<u32x4*>(&Vs[rr * C::VST + cc * 8]) = vr[it];
      }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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
    // every lane's transpose reads must land before the next tile overwrites the buffer
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // partial results: {m, l} per row, then the unnormalised output row
  const float lt = row_sum<MF>(l);
  if (!row_ok) return;
  const size_t prow = ((size_t)(b * a.Hkv + hkv) * a.nsplit + split) * a.rows + r;
  const size_t total_rows = (size_t)a.B * a.Hkv * a.nsplit * a.rows;
  float* pml = a.part + prow * 4;                 // {m, l} in a 16-byte slot
  float* po = a.part + total_rows * 4 + prow * DV;
  if (kg == 0) {
    pml[0] = m;
    pml[1] = lt;
  }
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < ACC / 4; ++g4) {
      const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
      if (dv < DV) {
        const f32x4 st = {o[db][g4 * 4 + 0], o[db][g4 * 4 + 1], o[db][g4 * 4 + 2], o[db][g4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(po + dv) = st;
      }
    }
}

// One workgroup (64 lanes) per (query row, kv head, batch item); lanes stride
// over the value columns in groups of four.
template <class E, int DV>
__global__ void __launch_bounds__(64) decode_reduce_kernel(FwdArgs a) {
  const int r = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = hkv * a.group + r / a.Lq;
  const int iq = r % a.Lq;
  const size_t pair = (size_t)(b * a.Hkv + hkv);
  const size_t total_rows = (size_t)a.B * a.Hkv * a.nsplit * a.rows;
  const float* pml = a.part;
  const float* po = a.part + total_rows * 4;

  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? half_to_f32<E>(((const uint16_t*)a.sinks)[h]) * kLog2e : -INFINITY;
  float M = sink2;
  for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, pml[((pair * a.nsplit + sp) * a.rows + r) * 4]);

  uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV;
  for (int dv = lane * 4; dv < DV; dv += 256) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
      if (has_sink) L = fast_exp2(sink2 - M);
      for (int sp = 0; sp < a.nsplit; ++sp) {
        const size_t prow = (pair * a.nsplit + sp) * a.rows + r;
        const float ms = pml[prow * 4];
        if (ms == -INFINITY) continue;
        const float f = fast_exp2(ms - M);
        L += pml[prow * 4 + 1] * f;
        const f32x4 x = *reinterpret_cast<const f32x4*>(po + prow * DV + dv);
        acc += x * f;
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const u32x2 st = {pack2<E>(acc[0] * inv, acc[1] * inv), pack2<E>(acc[2] * inv, acc[3] * inv)};
    st_global8(op + dv, st);
  }
}

}  // namespace sdpa
