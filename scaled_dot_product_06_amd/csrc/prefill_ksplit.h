// Prefill for 16-bit inputs with heads of 192 or 256 columns, (192,192), (192,128)
// and (256,256) (every grid, every mask kind), and heads up to 128 wide, (64,64),
// (80,80), (96,96), (128,128) and (96,64), on grids too small for the pipelined
// 32-row kernel (128-wide heads with an additive mask on every grid): the
// tiled online-softmax walk of lattice-inference
// "src/attention/flash.rs" (run_tiled_attention_head), with the bottom-right
// causal alignment of nuvec-core "tests/fast.rs"
// (attention_fallback_matches_a_direct_formula), laid out for gfx950:
//
//  * each wavefront owns 16 query rows of one head (16x16x32 MFMA tiles), so
//    its query fragment (32 registers) and output (64) leave room for two
//    wavefronts per SIMD, where a 32-row wavefront would hold its SIMD alone;
//  * the workgroup's eight wavefronts are four (head, row block) slots times
//    two key lanes. The workgroup walks the keys in 64-key steps; in each,
//    key lane j takes keys [32j, 32j + 32) of the step, so every wavefront
//    keeps its own online-softmax state over half of the keys, and at the end
//    the two lanes of a slot merge (m, l, O) in LDS with the log-sum-exp
//    combine. A workgroup thus covers 16 rows of four heads with two
//    wavefronts on each SIMD, and a 1024-row, 16-head call fills 256 compute
//    units;
//  * K and V steps go from global memory straight into LDS
//    (global_load_lds_dwordx4) through two double-buffered rings (K and V,
//    32 KB per step each at 256-wide heads, 128 KB in all; half that at 128;
//    192-wide rows sit in 256-wide ones, whose spare slots take a real chunk
//    of the row again, so every byte an operand read touches holds input data):
//    the K of step t+2 and the V of step
//    t+1 are loaded while step t runs, one barrier per step;
//  * the walk is software-pipelined inside each wavefront: the QK^T MFMAs of
//    step t+1 are issued among the exponentials of step t, and the PV MFMAs of
//    step t among the row maxima of step t+1;
//  * tiles some row sees only in part (the causal diagonal, a window's edge, a
//    ragged end) have their hidden scores set to -inf and their row maxima
//    taken again, at the top of their step. A boolean mask is read as the
//    caller's bytes, staged through a small LDS ring, and enters the scores as
//    the MFMA accumulators' starting values, 0 or -inf, so its steps need no
//    masking pass. An additive mask goes through a ring
//    of its own in the order the lanes read it and is added as the scores are
//    scaled, once per step;
//  * LDS rows hold their 16-byte chunks permuted by an XOR of the row index,
//    different for K (16 consecutive rows, one chunk each per read) and V
//    (16 rows, two adjacent chunks each per transposed read), so reads spread
//    over all banks.
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int D, int DV>
struct KsplitCfg {
  static constexpr int MF = 16, KW = 32, ACC = 4, KG = 4;
  static constexpr int ROWS = 16;              // query rows per wavefront
  static constexpr int SUB = 32;               // keys per wavefront per step
  static constexpr int KL = kKsplitLanes;      // key lanes
  static constexpr int BN = KL * SUB;          // keys per step
  static constexpr int NWH = kPrefillWaves;    // (head, row block) slots per workgroup
  static constexpr int NW = NWH * KL;          // wavefronts per workgroup
  // LDS row widths (elements) of K and of V: 192-wide rows sit in 256-wide ones
  static constexpr int LW = D <= 64 ? 64 : D <= 128 ? 128 : 256;       // K
  static constexpr int LWV = DV <= 64 ? 64 : DV <= 128 ? 128 : 256;   // V
  static constexpr int RB = LW * 2, RBV = LWV * 2;      // bytes per LDS row
  static constexpr int CPR = LW / 8, CPRV = LWV / 8;    // 16-byte chunks per LDS row
  static constexpr int KCH = D / 8, VCH = DV / 8;       // real chunks of a K and a V row
  static constexpr int ROWS_PER_KB = 1024 / RB, ROWS_PER_KB_V = 1024 / RBV;
  static constexpr int TILE_BYTES = BN * RB, TILE_BYTES_V = BN * RBV;   // one step of K, of V
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / NW;       // direct loads per step
  static constexpr int LOADS_PER_WAVE_V = TILE_BYTES_V / 1024 / NW;
  static constexpr int NQC = (D + KW - 1) / KW;  // QK^T k-steps (an 80-wide query is zero past 80)
  static constexpr int NSB = SUB / MF;         // 16-key blocks per wavefront step
  static constexpr int NDB = DV / MF;          // 16-column output blocks
  static constexpr int NPK = SUB * MF / 64 / 2;  // packed weight pairs per lane
  static_assert((D == DV && (D == 64 || D == 80 || D == 96 || D == 128 || D == 192 || D == 256)) ||
                    (D == 96 && DV == 64) || (D == 192 && DV == 128),
                "the key-split prefill serves (64,64), (80,80), (96,96), (128,128), (192,192), (256,256), "
                "(96,64) and (192,128)");
  static_assert(D % 8 == 0 && DV % MF == 0, "whole 16-byte query groups and 16-column output blocks");
  static_assert(2 * NDB * 64 * 16 <= TILE_BYTES, "two slots' merge partials fit one K stage");
  static_assert(TILE_BYTES_V % (1024 * NW) == 0, "loads divide among wavefronts");
  static_assert(NSB == 2 && NPK == 4, "two 16-key blocks make one 32-key PV step");
};

// K: the chunk of row r sits at slot chunk ^ (r % CPR) (CPR = 32 chunks per row in
// the 256-wide layout, 16 in the 128-wide one); the 16 rows one read touches (r0 .. r0+15, r0 a
// multiple of 16) land on 16 different slots. At 64-wide heads two 128-byte rows
// share a 256-byte line of banks, so the XOR is (r / 2) % 8: the 16 rows take the
// two halves of the line times 8 different slots.
template <int LW> __device__ __forceinline__ int ks_swz_k(int row) {
  return LW == 64 ? (row >> 1) % 8 : row % (LW / 8);
}
// V: pairs of chunks move together (XOR by an even number), by 2 * (r % 8); each
// half-wavefront of a transposed read covers 8 consecutive rows, whose 8
// different pairs fill one 256-byte line of banks. At 64-wide heads (four pairs
// per row, two rows per line) by 2 * ((r / 2) % 4): 2 row halves times 4 pairs.
template <int LW> __device__ __forceinline__ int ks_swz_v(int row) {
  return LW == 64 ? 2 * ((row >> 1) % 4) : 2 * (row % 8);
}
// the chunk a lane loads into layout slot `slot` of a row with REAL chunks (a
// row narrower than its layout): slots past the real ones take a real chunk again
template <int CPR, int REAL> __device__ __forceinline__ int ks_src_chunk(int slot) {
  if constexpr (REAL < CPR) return slot < REAL ? slot : slot - REAL;
  return slot;
}

// bytes between rows of the boolean-mask ring (64 keys plus padding)
constexpr int kMaskRow = 80;
// mask modes of the kernel
constexpr int kKsPlain = 0, kKsBool = 1, kKsAdd = 2;

// s_waitcnt immediate: vmcnt(n) only (gfx9 encoding, the other counters left at their maxima)
constexpr int ks_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate: lgkmcnt(0) only
constexpr int ks_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

// permlane16_swap(x, x) leaves in every lane the values of the two 16-lane rows
// of its pair: {even row, odd row}; so the pair reduction is over lanes l, l^16.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MK: kKsPlain (no mask or causal), kKsBool (boolean mask bytes) or kKsAdd
// (additive mask values)
template <class E, int D, int DV, int MK>
__global__ void __launch_bounds__((KsplitCfg<D, DV>::NW * 64)) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_ksplit_kernel(FwdArgs a) {
  using C = KsplitCfg<D, DV>;
  constexpr int MF = C::MF, BN = C::BN, SUB = C::SUB;
  using acc_t = f32x4;
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[C::TILE_BYTES_V];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[C::TILE_BYTES_V];
  __shared__ float merge_ml[C::NWH][2][MF];
  // boolean mask ring: up to 64 rows x 64 keys per stage, rows 80 bytes apart so
  // that the 16 rows x 4 groups one wavefront reads fall on 64 different banks
  constexpr bool BOOLMASK = MK == kKsBool, ADDMASK = MK == kKsAdd;
  __shared__ __attribute__((aligned(16))) uint8_t mstage[2][BOOLMASK ? C::NWH * 16 * kMaskRow : 16];
  // additive mask ring: per (slot, key lane) 64 lanes x 8 values, in the order
  // each lane reads them (one 16-byte read per lane and step)
  __shared__ __attribute__((aligned(16))) uint8_t astage[2][ADDMASK ? C::NWH * C::KL * 1024 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kl = w / C::NWH;          // key lane
  const int ws = w % C::NWH;          // (head, row block) slot
  const int col = lane % MF;          // query within the wavefront's rows
  const int kg = lane / MF;           // k-group (4 of them)

  const int heads = a.Hq * a.B / a.head_blocks;
  const int wph = C::NWH / heads;
  const int bm = wph * C::ROWS;
  int hb, qb;
  prefill_item((int)blockIdx.x, a.head_blocks, a.nqb, a.group / heads, hb, qb);
  const int groups_per_b = a.Hq / heads;
  const int b = hb / groups_per_b;
  const int h0 = (hb % groups_per_b) * heads;
  const int hkv = h0 / a.group;
  const int h = h0 + ws / wph;
  const int wi0 = qb * bm + (ws % wph) * C::ROWS;
  const int shift = a.Lk - a.Lq;

  // keys the workgroup needs ([kbeg, kend)), in steps tb .. tb + ntiles - 1
  int kend = a.Lk;
  if (a.mask_kind == kMaskCausal) kend = min(a.Lk, min(qb * bm + bm, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  int kbeg = 0;
  if (a.window > 0) kbeg = min(max(0, qb * bm + shift - a.window + 1), kend);
  const int tb = kbeg / BN;
  const int ntiles = max((kend + BN - 1) / BN - tb, 0);
  // keys every row of this wavefront sees: [w_klo, w_kfull)
  int w_kfull = a.Lk;
  if (a.mask_kind == kMaskCausal) w_kfull = min(a.Lk, wi0 + shift + 1);
  int w_klo = 0;
  if (a.window > 0) w_klo = min(wi0 + C::ROWS, a.Lq) - 1 + shift - a.window + 1;

  const int iq = wi0 + col;
  u32x4 qop[C::NQC];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      bool in = iq < a.Lq;
      // (the k-step past an 80-wide query's end reads zeros: its K operands are
      // real chunks loaded again, so it adds nothing to the scores)
      if constexpr (D % C::KW != 0) in = in && c * C::KW + kg * 8 < D;
      if (in) x = ld_global16(qp + c * C::KW + kg * 8);
      qop[c] = x ^ a.qsign;
    }
  }

  // Boolean mask, read as the caller's bytes. The workgroup's bm rows x 64 keys
  // of a step (16 rows per loader wavefront, lane l: row l / 4, keys 16 (l % 4)
  // .. +15, one 16-byte load; global memory is accessed in unaligned mode, so a
  // group may start at any byte) go through a two-stage LDS ring: loaded into
  // registers three steps before the step whose scores use them, written to
  // the ring at the next step, read after that step's barrier. One load per
  // loader lane and step keeps the per-step address traffic to a few cache
  // lines per row. Keys at or past Lk read as hidden.
  const bool mloader = BOOLMASK && w < wph;
  const uint8_t* mload_row =
      mloader ? a.mask + (size_t)min(qb * bm + w * 16 + lane / 4, a.Lq - 1) * a.Lk : nullptr;
  auto mask_chunk = [&](int step) -> u32x4 {
    const int key = step * BN + 16 * (lane % 4);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key + 16 <= a.Lk) {
      __builtin_memcpy(&x, mload_row + key, 16);
    } else {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
      for (int j = 0; j < 16 && key + j < a.Lk; ++j) wv[j / 4] |= (uint32_t)mload_row[key + j] << (8 * (j % 4));
      x = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    return x;
  };
  auto mask_store = [&](int stage, u32x4 x) {
    *reinterpret_cast<u32x4*>(&mstage[stage][(w * 16 + lane / 4) * kMaskRow + (lane % 4) * 16]) = x;
  };
  // the lane's bytes of a step: row (slot row block) + col, keys 32 kl + 4 kg (+16)
  const int mrd = ((ws % wph) * 16 + col) * kMaskRow + SUB * kl + 4 * kg;
  auto mask_read = [&](int stage) -> u32x2 {
    return u32x2{*reinterpret_cast<const uint32_t*>(&mstage[stage][mrd]),
                 *reinterpret_cast<const uint32_t*>(&mstage[stage][mrd + 16])};
  };
  // The scores of a step start from its mask: each accumulator starts at 0
  // (visible) or -inf (hidden), so the MFMAs yield the masked scores and the
  // step needs no separate masking pass.
  u32x4 mpend = {0u, 0u, 0u, 0u};   // a loader lane's chunk, waiting for its ring stage

  // Additive mask: key lane 0's wavefront of each slot loads the slot's 16 rows x
  // 64 keys of a step (two 16-byte loads per lane: 8 keys of one row each) three
  // steps ahead, and writes them to the ring at the next step in the order the
  // readers take them: lane (col, kg) of key lane kl gets keys 4 kg .. 4 kg + 3 and
  // 16 + 4 kg .. of its 32. Keys at or past Lk read as -inf. The scores are then
  // scaled once with the mask added, in base 2, and used unscaled after that.
  const bool aloader = ADDMASK && kl == 0;
  const uint16_t* arow[2] = {nullptr, nullptr};
  if (aloader) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rq = (lane + 64 * j) / 8;   // row of the slot's 16
      arow[j] = (const uint16_t*)a.amask + b * a.ms[0] + h * a.ms[1] + (int64_t)min(wi0 + rq, a.Lq - 1) * a.ms[2];
    }
  }
  auto add_chunk = [&](int step, int j) -> u32x4 {
    const int key = step * BN + 8 * ((lane + 64 * j) % 8);
    u32x4 x;
    if (key + 8 <= a.Lk) {
      __builtin_memcpy(&x, arow[j] + key, 16);
    } else {
      uint32_t hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = key + e < a.Lk ? arow[j][key + e] : neg_inf_bits<E>();
      x = u32x4{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
    }
    return x;
  };
  // 8-key group g of a row (keys 8g .. 8g+7 of the step): key lane g / 4, block
  // nb = (g % 4) / 2, halves to the lanes of k-groups 2 (g % 2) and 2 (g % 2) + 1
  auto add_store = [&](int stage, int j, u32x4 x) {
    const int q = lane + 64 * j, row = q / 8, g = q % 8;
    const int kk = g / 4, nb = (g % 4) / 2, kg0 = 2 * (g % 2);
    uint8_t* base = &astage[stage][(ws * C::KL + kk) * 1024 + nb * 8];
    *reinterpret_cast<u32x2*>(base + (kg0 * 16 + row) * 16) = u32x2{x[0], x[1]};
    *reinterpret_cast<u32x2*>(base + ((kg0 + 1) * 16 + row) * 16) = u32x2{x[2], x[3]};
  };
  auto add_read = [&](int stage) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(&astage[stage][((ws * C::KL + kl) * 64 + lane) * 16]);
  };
  // scores scaled once, mask added: s = c s + mask log2(e)
  auto add_apply = [&](acc_t (&s)[C::NSB], u32x4 mv) {
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < C::ACC; ++i) {
        const uint32_t wv = mv[nb * 2 + i / 2];
        const float add = half_to_f32<E>((uint16_t)((i & 1) ? (wv >> 16) : (wv & 0xFFFFu))) * kLog2e;
        s[nb][i] = fmaf(s[nb][i], a.c, add);
      }
  };
  u32x4 apend[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  // scale applied to the scores from here on (1 once the additive mask's pass scaled them)
  const float cs = ADDMASK ? 1.0f : a.c;
  auto score_init = [&](acc_t (&s)[C::NSB], u32x2 mb) {
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      if constexpr (BOOLMASK) {
        // bit 8i of y: byte i (key 16 nb + 4 kg + i) is nonzero
        uint32_t y = mb[nb];
        y |= y >> 4;
        y |= y >> 2;
        y |= y >> 1;
#pragma unroll
        for (int i = 0; i < C::ACC; ++i) s[nb][i] = keep_if_bit(0.0f, y, 8 * i);
      } else {
        s[nb] = acc_t{};
      }
    }
  };

  acc_t o[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) o[d] = acc_t{};
  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? half_to_f32<E>(((const uint16_t*)a.sinks)[h]) * kLog2e : 0.0f;
  float m = has_sink ? sink2 : -INFINITY;
  float l = 0.0f, tmax = -INFINITY;

  const uint8_t* kbase = (const uint8_t*)a.k + (b * a.ks[0] + hkv * a.ks[1]) * 2;
  const uint8_t* vbase = (const uint8_t*)a.v + (b * a.vs[0] + hkv * a.vs[1]) * 2;
  const uint32_t krs = (uint32_t)(a.ks[2] * 2), vrs = (uint32_t)(a.vs[2] * 2);

  // direct loads: the lane's 16-byte chunk of rows (w + NW*it) * ROWS_PER_KB + lane / CPR
  uint32_t offk[C::LOADS_PER_WAVE], offv[C::LOADS_PER_WAVE_V];
  int ldrow[C::LOADS_PER_WAVE], ldrowv[C::LOADS_PER_WAVE_V];
#pragma unroll
  for (int it = 0; it < C::LOADS_PER_WAVE; ++it) {
    const int row = (w + C::NW * it) * C::ROWS_PER_KB + lane / C::CPR;
    ldrow[it] = row;
    offk[it] = row * krs + ks_src_chunk<C::CPR, C::KCH>((lane % C::CPR) ^ ks_swz_k<C::LW>(row)) * 16;
  }
#pragma unroll
  for (int it = 0; it < C::LOADS_PER_WAVE_V; ++it) {
    const int row = (w + C::NW * it) * C::ROWS_PER_KB_V + lane / C::CPRV;
    ldrowv[it] = row;
    offv[it] = row * vrs + ks_src_chunk<C::CPRV, C::VCH>((lane % C::CPRV) ^ ks_swz_v<C::LWV>(row)) * 16;
  }
  // rows past the last key read the last key's row instead (their weights are
  // zero); a step starts at most at Lk - 1, so the unsigned offsets stay >= 0
  auto tail_over = [&](int k0, int row) -> uint32_t { return (uint32_t)max(k0 + row - (a.Lk - 1), 0); };
  auto issue_k = [&](int step, uint8_t* dst) {
    const int k0 = step * BN;
    const uint8_t* kt = kbase + (size_t)k0 * krs;
    const bool tail = k0 + BN > a.Lk;
#pragma unroll
    for (int it = 0; it < C::LOADS_PER_WAVE; ++it) {
      uint32_t ok = offk[it];
      if (tail) ok -= tail_over(k0, ldrow[it]) * krs;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + ok),
                                       (__attribute__((address_space(3))) void*)(dst + (w + C::NW * it) * 1024), 16,
                                       0, 0);
    }
  };
  auto issue_v = [&](int step, uint8_t* dst) {
    const int k0 = step * BN;
    const uint8_t* vt = vbase + (size_t)k0 * vrs;
    const bool tail = k0 + BN > a.Lk;
#pragma unroll
    for (int it = 0; it < C::LOADS_PER_WAVE_V; ++it) {
      uint32_t ov = offv[it];
      if (tail) ov -= tail_over(k0, ldrowv[it]) * vrs;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + ov),
                                       (__attribute__((address_space(3))) void*)(dst + (w + C::NW * it) * 1024), 16,
                                       0, 0);
    }
  };

  // K operand of key block nb, k-step c: row SUB*kl + 16 nb + col, chunk 4c + kg.
  // With the row's XOR (16 nb + col), the four k-steps c and c + 4 and the two
  // blocks differ by constants, so four lane offsets serve all sixteen reads.
  constexpr int KC = C::NQC < 4 ? C::NQC : 4;   // k-steps per group of K operand reads
  uint32_t kb4[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c)
    kb4[c] = (SUB * kl + col) * C::RB + (((4 * c + kg) ^ ks_swz_k<C::LW>(SUB * kl + col)) * 16);
  // (at 64- and 128-wide heads the XOR of row 16 nb + col does not depend on nb:
  // the blocks differ by 16 rows)
  auto k_off = [&](int c, int nb) -> uint32_t {
    if constexpr (C::LW <= 128) return kb4[c] + nb * (16 * C::RB);
    return c < 4 ? kb4[c] + nb * (16 * C::RB + 256) : kb4[c - 4] + 256 + nb * (16 * C::RB - 256);
  };
  // V^T operand of output block db: transposed reads of keys 4g..4g+3 and
  // 16+4g..16+4g+3 (g = lane / 16); provider lane l points at row
  // SUB*kl + l/4 (+16), columns 16 db + 4 (l % 4) .. +3. The V XOR pairs chunk
  // 2 db with row % 8, so blocks db and db + 8 (256-wide heads) differ by 256 bytes.
  const int vr = lane >> 2;
  constexpr int VB = C::NDB < 8 ? C::NDB : 8;   // output blocks per group of V^T reads
  uint32_t vb8[VB];
  const int vsw = ks_swz_v<C::LWV>(SUB * kl + vr) / 2;   // the row's pair XOR (the same 16 rows on)
#pragma unroll
  for (int db = 0; db < VB; ++db)
    vb8[db] = (SUB * kl + vr) * C::RBV + ((2 * (db ^ vsw) + ((lane >> 1) & 1)) * 16) + (lane & 1) * 8;
  auto v_off = [&](int db) -> uint32_t { return db < VB ? vb8[db] : vb8[db - VB] + 256; };
  static_assert(C::NQC <= 8 && C::NDB <= 16 && (C::LW == 256 || C::NQC <= 4) && (C::LWV == 256 || C::NDB <= 8),
                "LDS operands come in up to two groups of up to four k-steps and eight blocks");

  // LDS operands go through two register buffers of eight 16-byte groups: the
  // reads of one group are issued before the MFMAs of the previous one, and an
  // explicit wait for all LDS reads follows those MFMAs. (With direct-to-LDS loads
  // in flight every LDS wait is a wait for all reads, so this keeps each wait
  // behind a group of MFMAs instead of in front of each one.)
  // (a group stops at the last k-step or block: 192-wide heads take a second K group
  // of two k-steps, 192-wide values a second V group of four blocks)
  auto read_k = [&](const uint8_t* Ks, int c0, u32x4 (&buf)[8]) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      if (c0 + c < C::NQC)
#pragma unroll
        for (int nb = 0; nb < C::NSB; ++nb) buf[c * 2 + nb] = *reinterpret_cast<const u32x4*>(Ks + k_off(c0 + c, nb));
  };
  auto mma_qk = [&](int c0, const u32x4 (&buf)[8], acc_t (&s)[C::NSB]) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      if (c0 + c < C::NQC)
#pragma unroll
        for (int nb = 0; nb < C::NSB; ++nb) s[nb] = mma16<E, MF>(buf[c * 2 + nb], qop[c0 + c], s[nb]);
  };
  auto read_v = [&](const uint8_t* Vs, int db0, u32x4 (&buf)[8]) {
#pragma unroll
    for (int d = 0; d < VB; ++d) {
      if (db0 + d >= C::NDB) continue;
      const u32x2 ra = lds_read_tr16((const uint16_t*)(Vs + v_off(db0 + d)));
      const u32x2 rb = lds_read_tr16((const uint16_t*)(Vs + v_off(db0 + d) + 16 * C::RBV));
      buf[d] = u32x4{ra[0], ra[1], rb[0], rb[1]};
    }
  };
  auto lds_wait = [] { __builtin_amdgcn_s_waitcnt(ks_lgkm0()); };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // S^T = K Q^T for the wavefront's 32 keys of one step (not pipelined: the prologue)
  auto qk = [&](const uint8_t* Ks, acc_t (&s)[C::NSB]) {
    u32x4 ba[8], bb[8];
    u32x2 mb = {0u, 0u};
    if constexpr (BOOLMASK) mb = mask_read(0);
    read_k(Ks, 0, ba);
    lds_wait();
    score_init(s, mb);
    if constexpr (C::NQC > 4) {
      read_k(Ks, 4, bb);
      lds_wait();
    }
    mma_qk(0, ba, s);
    if constexpr (C::NQC > 4) mma_qk(4, bb, s);
  };
  auto row_max16 = [](float x) { return max_xor16(max_xor32(x)); };
  auto tile_max_full = [&](acc_t (&s)[C::NSB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < C::ACC; ++i) mx = fmaxf(mx, s[nb][i]);
    tmax = row_max16(mx) * cs;
  };
  // the lane's scores sit at keys k0 + 16 nb + 4 kg + i of the step's sub-tile
  // (causal and window limits, and keys past Lk; a boolean mask is already in the scores)
  auto tile_max_masked = [&](int step, acc_t (&s)[C::NSB]) {
    const int k0 = step * BN + SUB * kl;
    const bool row_ok = iq < a.Lq;
    const int lim = a.mask_kind == kMaskCausal ? min(iq + shift, a.Lk - 1) : a.Lk - 1;
    const int lo = a.window > 0 ? iq + shift - a.window : -1;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < C::ACC; ++i) {
        const int key = k0 + 16 * nb + 4 * kg + i;
        const bool vis = row_ok & (key <= lim) & (key > lo);
        s[nb][i] = vis ? s[nb][i] : -INFINITY;
      }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < C::ACC; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = row_max16(mx);
    tmax = (mx == -INFINITY) ? -INFINITY : mx * cs;
  };
  // weights rounded to 16 bits; the running sum adds the same rounded weights
  auto weights = [&](acc_t (&s)[C::NSB], uint32_t (&pk)[C::NPK]) {
    const float mu = (m == -INFINITY) ? 0.0f : m;
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
      for (int i = 0; i < C::ACC; i += 2) {
        const float p0 = fast_exp2(fmaf(s[nb][i], cs, -mu));
        const float p1 = fast_exp2(fmaf(s[nb][i + 1], cs, -mu));
        pk[nb * 2 + i / 2] = pack2<E>(p0, p1);
      }
    float l0 = pair_sum<E>(pk[0], 0.0f), l1 = pair_sum<E>(pk[1], 0.0f);
    l0 = pair_sum<E>(pk[2], l0);
    l1 = pair_sum<E>(pk[3], l1);
    l += l0 + l1;
  };
  // O^T += V^T P^T: MFMA k-slot 8g + e is key 4g + e (e < 4) or 16 + 4g + e - 4
  auto mma_pv = [&](int db0, const u32x4 (&buf)[8], const uint32_t (&pk)[C::NPK]) {
    const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
    for (int d = 0; d < VB; ++d)
      if (db0 + d < C::NDB) o[db0 + d] = mma16<E, MF>(buf[d], pb, o[db0 + d]);
  };

  acc_t sa[C::NSB], sb[C::NSB];
  uint32_t pk[C::NPK];
  // Step t: the loads of step t+1's K and step t's V have landed (they were the
  // last issued, so vmcnt(0)), and after the barrier every wavefront is done
  // with step t-1, so K stage t%2 (held K(t), scored in step t-1) and V stage
  // (t+1)%2 (held V(t-1)) take K(t+2) and V(t+1).
  auto step = [&](int t, acc_t (&scur)[C::NSB], acc_t (&snext)[C::NSB], const uint8_t* Knext, uint8_t* Kload,
                  const uint8_t* Vcur, uint8_t* Vload) {
    __builtin_amdgcn_s_waitcnt(ks_vmcnt(0));
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the mask of step t + 2 into ring stage t % 2 (last read for step t's scores)
    if (mloader) mask_store(t & 1, mpend);
    if (t + 2 < ntiles) issue_k(tb + t + 2, Kload);
    if (t + 1 < ntiles) issue_v(tb + t + 1, Vload);
    if (mloader && t + 3 < ntiles) mpend = mask_chunk(tb + t + 3);
    if constexpr (ADDMASK) {
      if (aloader) {
        add_store(t & 1, 0, apend[0]);
        add_store(t & 1, 1, apend[1]);
        if (t + 3 < ntiles) {
          apend[0] = add_chunk(tb + t + 3, 0);
          apend[1] = add_chunk(tb + t + 3, 1);
        }
      }
    }
    const int kt = tb + t;
    const int k0 = kt * BN + SUB * kl;
    if (k0 + SUB > w_kfull || k0 < w_klo) tile_max_masked(kt, scur);
    softmax_rebase<C::NDB>(tmax, m, l, o);
    u32x4 ba[8], bb[8];
    u32x2 mb = {0u, 0u};
    u32x4 mv = {0u, 0u, 0u, 0u};
    fence();
    if constexpr (BOOLMASK) mb = mask_read((t + 1) & 1);
    if constexpr (ADDMASK) mv = add_read((t + 1) & 1);
    read_k(Knext, 0, ba);
    weights(scur, pk);
    fence();
    lds_wait();
    if constexpr (C::NQC > 4) {
      // 192- and 256-wide heads: two groups of K operands and up to two of V,
      // each group's reads issued before the MFMAs of the previous one
      read_k(Knext, 4, bb);
      score_init(snext, mb);
      fence();
      // the MFMA groups at raised wave priority: of the two wavefronts on a SIMD,
      // which leave each barrier together, the one in its MFMA groups issues first
      __builtin_amdgcn_s_setprio(1);
      mma_qk(0, ba, snext);
      fence();
      lds_wait();
      read_v(Vcur, 0, ba);
      fence();
      mma_qk(4, bb, snext);
      fence();
      lds_wait();
      read_v(Vcur, 8, bb);
      fence();
      mma_pv(0, ba, pk);
      fence();
      lds_wait();
      mma_pv(8, bb, pk);
      fence();
    } else {
      // 64- and 128-wide heads: one group of K operands and one of V
      read_v(Vcur, 0, bb);
      score_init(snext, mb);
      fence();
      __builtin_amdgcn_s_setprio(1);
      mma_qk(0, ba, snext);
      fence();
      lds_wait();
      mma_pv(0, bb, pk);
      fence();
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (ADDMASK) add_apply(snext, mv);
    tile_max_full(snext);
  };

  // prologue: the mask of steps 0 and 1 into the ring and step 2's in registers;
  // K(0), V(0), K(1) in flight; step 0's scores from K(0)
  if (mloader) {
    const u32x4 m0 = ntiles > 0 ? mask_chunk(tb) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 m1 = ntiles > 1 ? mask_chunk(tb + 1) : u32x4{0u, 0u, 0u, 0u};
    if (ntiles > 2) mpend = mask_chunk(tb + 2);
    mask_store(0, m0);
    mask_store(1, m1);
  }
  if constexpr (ADDMASK) {
    if (aloader) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 a0 = ntiles > 0 ? add_chunk(tb, j) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 a1 = ntiles > 1 ? add_chunk(tb + 1, j) : u32x4{0u, 0u, 0u, 0u};
        if (ntiles > 2) apend[j] = add_chunk(tb + 2, j);
        add_store(0, j, a0);
        add_store(1, j, a1);
      }
    }
  }
  if (ntiles > 0) {
    issue_k(tb, ks0);
    issue_v(tb, vs0);
  }
  if (ntiles > 1) issue_k(tb + 1, ks1);
  if (ntiles > 1) {
    __builtin_amdgcn_s_waitcnt(ks_vmcnt(C::LOADS_PER_WAVE + C::LOADS_PER_WAVE_V));
  } else {
    __builtin_amdgcn_s_waitcnt(ks_vmcnt(0));
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ntiles > 0) {
    qk(ks0, sa);
    if constexpr (ADDMASK) add_apply(sa, add_read(0));
    tile_max_full(sa);
  }
  // even steps score into sb from K stage 1 and read V stage 0; odd steps the
  // reverse. The last step also scores a next tile from a stage holding stale
  // (or never loaded) data and discards it.
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa, sb, ks1, ks0, vs0, vs1);
    if (t + 1 >= ntiles) break;
    step(t + 1, sb, sa, ks0, ks1, vs1, vs0);
  }

  // merge the two key lanes of each slot: lane 1 leaves (m, l, O) in LDS (the
  // K ring, free once every wavefront has passed this barrier), lane 0 combines
  __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  l = sum_xor16(sum_xor32(l));
  f32x4* part = reinterpret_cast<f32x4*>(ws < 2 ? ks0 : ks1) + (ws % 2) * (C::NDB * 64);
  if (kl == 1) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) part[db * 64 + lane] = o[db];
    if (kg == 0) {
      merge_ml[ws][0][col] = m;
      merge_ml[ws][1][col] = l;
    }
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (kl == 1 || wi0 >= a.Lq) return;
  const float m1 = merge_ml[ws][0][col], l1 = merge_ml[ws][1][col];
  const float mm = fmaxf(m, m1);
  const float f0 = m == -INFINITY ? 0.0f : fast_exp2(m - mm);
  const float f1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - mm);
  float lt = l * f0 + l1 * f1;
  if (has_sink) lt += fast_exp2(sink2 - mm);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (iq >= a.Lq) return;
  const float g0 = f0 * inv, g1 = f1 * inv;
  uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq) * DV;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    const f32x4 p = part[db * 64 + lane];
    const f32x4 r = o[db] * g0 + p * g1;
    const u32x2 st = {pack2<E>(r[0], r[1]), pack2<E>(r[2], r[3])};
    st_global8(op + db * MF + kg * 4, st);
  }
}

}  // namespace sdpa
