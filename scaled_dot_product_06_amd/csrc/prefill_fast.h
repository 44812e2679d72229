// Prefill for 16-bit inputs with D = Dv in {64, 128}: the same tiled
// online-softmax walk as prefill_kernel (lattice-inference
// "src/attention/flash.rs", run_tiled_attention_head; causal alignment of
// nuvec-core "tests/fast.rs"), laid out for gfx950 occupancy:
//
//  * K and V tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4: each lane's 16 bytes land at base + 16 * lane),
//    so no registers hold tile data and no LDS store instructions are issued;
//  * two LDS stages: tile t+1 streams in while tile t is computed, with one
//    workgroup barrier per tile; the stages are distinct LDS objects so the
//    compiler can tell the loads into one from the reads of the other;
//  * each LDS row is stored with its 16-byte chunks permuted by an XOR of the
//    row index (different for K and V), chosen so that the K-operand reads
//    (16 consecutive rows, one chunk each) and the V transpose reads (8
//    consecutive rows, four chunks each) touch every bank equally;
//  * the register budget is held to two wavefronts per SIMD, so one
//    wavefront's softmax arithmetic overlaps the other's MFMA work.
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int D>
struct FastCfg {
  static constexpr int MF = 32, KW = 16, ACC = 16, KG = 2;
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int NW = 4;                  // wavefronts per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int RB = D * 2;              // bytes per row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int ROWS_PER_KB = 1024 / RB; // rows filled by one direct-load instruction
  static constexpr int TILE_BYTES = BN * RB;    // one K or V tile
  static constexpr int LOADS = TILE_BYTES / 1024;  // direct-load instructions per tile and tensor
  static constexpr int LOADS_PER_WAVE = LOADS / NW;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K then V
  static constexpr int NQC = D / KW;
  static constexpr int NSB = BN / MF;
  static constexpr int NPV = BN / KW;
  static constexpr int NDB = D / MF;
  static_assert(D == 64 || D == 128, "fast prefill covers 64- and 128-wide heads");
  static_assert(LOADS % NW == 0, "loads divide among wavefronts");
};

// chunk permutations (XOR masks) for the K and V tiles
template <int D> __device__ __forceinline__ int swz_k(int row) { return row % FastCfg<D>::CPR; }
template <int D> __device__ __forceinline__ int swz_v(int row) {
  return 4 * ((row / (256 / FastCfg<D>::RB)) % (FastCfg<D>::CPR / 4));
}

template <class E, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_fast_kernel(FwdArgs a) {
  using C = FastCfg<D>;
  constexpr int MF = C::MF, ACC = C::ACC, BN = C::BN;
  using acc_t = f32x16;
  // Two stages as two distinct LDS objects: the compiler can then prove that
  // the direct loads into one stage never alias the reads of the other, and
  // does not make the reads of tile t wait for the loads of tile t+1.
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps control flow scalar
  const int col = lane % MF;
  const int kg = lane / MF;

  const int heads = a.Hq * a.B / a.head_blocks;
  const int wph = C::NW / heads;
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
  const int shift = a.Lk - a.Lq;

  int kend = a.Lk;
  if (a.mask_kind == kMaskCausal) kend = min(a.Lk, min(qb * bm + bm, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BN - 1) / BN;

  const bool wave_live = wi0 < a.Lq;
  const int w_last = min(wi0 + MF, a.Lq) - 1;
  int w_kend = a.Lk, w_kfull = a.Lk;
  if (a.mask_kind == kMaskCausal) {
    w_kend = min(a.Lk, w_last + shift + 1);
    w_kfull = min(a.Lk, wi0 + shift + 1);
  } else if (a.mask_kind == kMaskBool) {
    w_kfull = 0;
  }

  const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(b * a.Hq + h) * a.Lq + iq) * D;
  u32x4 qop[C::NQC];
#pragma unroll
  for (int c = 0; c < C::NQC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (iq < a.Lq) x = ld_global16(qp + c * C::KW + kg * 8);
    qop[c] = x ^ a.qsign;
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

  const uint8_t* kbase = (const uint8_t*)a.k + (size_t)(b * a.Hkv + hkv) * (size_t)a.Lk * C::RB;
  const uint8_t* vbase = (const uint8_t*)a.v + (size_t)(b * a.Hkv + hkv) * (size_t)a.Lk * C::RB;
  const uint8_t* mrow = a.mask + (size_t)iq * a.Lk;

  // direct loads: per lane, byte offsets of its 16-byte chunk within the tile
  // (row blk*ROWS_PER_KB + lane/CPR, global chunk permuted by the row's XOR)
  const int ld_row = lane / C::CPR;
  const int ld_slot = lane % C::CPR;
  uint32_t offk[C::LOADS_PER_WAVE], offv[C::LOADS_PER_WAVE];
  int ldrow[C::LOADS_PER_WAVE];
#pragma unroll
  for (int it = 0; it < C::LOADS_PER_WAVE; ++it) {
    const int row = (w + C::NW * it) * C::ROWS_PER_KB + ld_row;
    ldrow[it] = row;
    offk[it] = row * C::RB + (ld_slot ^ swz_k<D>(row)) * 16;
    offv[it] = row * C::RB + (ld_slot ^ swz_v<D>(row)) * 16;
  }
  auto issue_tile = [&](int k0, uint8_t* sbase) {
    const uint8_t* kt = kbase + (size_t)k0 * C::RB;
    const uint8_t* vt = vbase + (size_t)k0 * C::RB;
    const bool tail = k0 + BN > a.Lk;
#pragma unroll
    for (int it = 0; it < C::LOADS_PER_WAVE; ++it) {
      uint32_t ok = offk[it], ov = offv[it];
      if (tail) {
        // rows past the end read the last real row instead; those keys get weight 0
        const int over = max(k0 + ldrow[it] - (a.Lk - 1), 0) * C::RB;
        ok -= over;
        ov -= over;
      }
      const int blk = w + C::NW * it;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + ok),
                                       (__attribute__((address_space(3))) void*)(sbase + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + ov),
                                       (__attribute__((address_space(3))) void*)(sbase + C::TILE_BYTES + blk * 1024),
                                       16, 0, 0);
    }
  };

  // transpose-read provider coordinates
  const int tr_e = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int tr_chunk = ((lane >> 4) & 1) * 2 + (tr_c >> 1);  // chunk within a 32-column block
  const int tr_half = (tr_c & 1) * 8;

  auto compute = [&](int t, const uint8_t* Ks) {
    const int k0 = t * BN;
    const bool full = k0 + BN <= w_kfull;
    const uint8_t* Vs = Ks + C::TILE_BYTES;

    acc_t s[C::NSB];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) s[nb] = acc_t{};
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) {
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb) {
        const int row = nb * MF + col;
        const u32x4 kop =
            *reinterpret_cast<const u32x4*>(Ks + row * C::RB + (((2 * c + kg) ^ swz_k<D>(row)) * 16));
        s[nb] = mma16<E, MF>(kop, qop[c], s[nb]);
      }
    }

    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) mx = fmaxf(mx, s[nb][i]);
    } else {
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) {
          const int key = k0 + nb * MF + acc_row<MF>(i, kg);
          bool vis = key < a.Lk && iq < a.Lq;
          if (a.mask_kind == kMaskCausal) vis = vis && key <= iq + shift;
          else if (a.mask_kind == kMaskBool) vis = vis && mrow[key] != 0;
          if (!vis) s[nb][i] = -INFINITY;
          mx = fmaxf(mx, s[nb][i]);
        }
    }
    mx = row_max<MF>(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * a.c;
    softmax_rebase<C::NDB>(tmax, m, l, o);
    const float mu = (m == -INFINITY) ? 0.0f : m;

    // weights, rounded to 16 bits for the MFMA; the running sum adds the same
    // rounded weights (two per v_dot2), so numerator and denominator agree
    uint32_t pk[C::NSB * ACC / 2];
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < ACC; i += 2) {
        const float p0 = fast_exp2(fmaf(s[nb][i], a.c, -mu));
        const float p1 = fast_exp2(fmaf(s[nb][i + 1], a.c, -mu));
        pk[(nb * ACC + i) / 2] = pack2<E>(p0, p1);
      }
    float lsum0 = 0.0f, lsum1 = 0.0f;
#pragma unroll
    for (int j = 0; j < C::NSB * ACC / 2; j += 2) {
      lsum0 = pair_sum<E>(pk[j], lsum0);
      lsum1 = pair_sum<E>(pk[j + 1], lsum1);
    }
    l += lsum0 + lsum1;

#pragma unroll
    for (int t8 = 0; t8 < C::NPV; ++t8) {
      const u32x4 pb = {pk[4 * t8], pk[4 * t8 + 1], pk[4 * t8 + 2], pk[4 * t8 + 3]};
      const int keyA = ((8 * t8) / ACC) * MF + acc_row<MF>((8 * t8) % ACC, kg) + tr_e;
      const int keyB = ((8 * t8 + 4) / ACC) * MF + acc_row<MF>((8 * t8 + 4) % ACC, kg) + tr_e;
      const uint8_t* vA = Vs + keyA * C::RB + tr_half;
      const uint8_t* vB = Vs + keyB * C::RB + tr_half;
      const int swA = swz_v<D>(keyA), swB = swz_v<D>(keyB);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int ch = db * 4 + tr_chunk;
        const u32x2 ra = lds_read_tr16((const uint16_t*)(vA + ((ch ^ swA) * 16)));
        const u32x2 rb = lds_read_tr16((const uint16_t*)(vB + ((ch ^ swB) * 16)));
        const u32x4 va = {ra[0], ra[1], rb[0], rb[1]};
        o[db] = mma16<E, MF>(va, pb, o[db]);
      }
    }
  };

  // one barrier per tile: tile t's loads have landed (own wait + barrier) and
  // every wavefront has finished tile t-1, whose stage the next loads reuse
  if (ntiles > 0) issue_tile(0, lds0);
  for (int t = 0; t < ntiles; t += 2) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) issue_tile((t + 1) * BN, lds1);
    if (wave_live && t * BN < w_kend) compute(t, lds0);
    if (t + 1 >= ntiles) break;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < ntiles) issue_tile((t + 2) * BN, lds0);
    if (wave_live && (t + 1) * BN < w_kend) compute(t + 1, lds1);
  }

  if (!wave_live) return;
  float lt = row_sum<MF>(l);
  if (has_sink) lt += fast_exp2(sink2 - m);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (iq >= a.Lq) return;
  uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * D;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < ACC / 4; ++g4) {
      const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
      const u32x2 st = {pack2<E>(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv),
                        pack2<E>(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv)};
      st_global8(op + dv, st);
    }
}

}  // namespace sdpa
