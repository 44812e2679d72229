// Prefill for 16-bit inputs with (D, Dv) in {(64, 64), (80, 80), (96, 96), (128, 128),
// (96, 64)}: the tiled online-softmax
// walk of lattice-inference "src/attention/flash.rs" (run_tiled_attention_head)
// with the bottom-right causal alignment of nuvec-core "tests/fast.rs"
// (attention_fallback_matches_a_direct_formula), laid out for gfx950:
//
//  * each wavefront owns one 32-row MFMA block of query rows and the
//    workgroup's four wavefronts share every K/V tile (one head each under
//    grouped queries). The kernel fits 168 registers and 48 KB of LDS, so
//    three workgroups share a compute unit and three wavefronts from
//    different workgroups share each SIMD, hiding each other's latencies;
//  * K and V tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4: each lane's 16 bytes land at base + 16 * lane),
//    through a ring of three stages, one tile ahead of the step that reads it,
//    one barrier per tile; the
//    stages are distinct LDS objects so the compiler can tell the loads into
//    one stage from the reads of another;
//  * the loop is software-pipelined inside each wavefront: the QK^T MFMAs of
//    tile t+1 are issued among the exponentials of tile t, and the PV MFMAs
//    of tile t among the row maxima of tile t+1, so the matrix cores and the
//    vector ALUs work at the same time;
//  * a tile some row sees only in part (the causal diagonal, a ragged end,
//    every tile under a boolean mask) has its hidden scores set to -inf and
//    its row maxima taken again at the top of its step; other tiles skip
//    that branch, so the pipelined body has a single path;
//  * each LDS row holds its 16-byte chunks permuted by an XOR of the row index
//    (different for K and V), so the K-operand reads (16 consecutive rows, one
//    chunk each) and the V transpose reads (8 consecutive rows, four chunks
//    each) touch every bank equally;
//  * 80- and 96-wide rows sit in the 128-wide LDS layout: the QK^T k-steps and
//    the PV output blocks cover the real columns (an 80-wide output's third
//    32-column block computes 16 spare columns that are never stored), and the
//    lanes whose layout slot falls past a row's real chunks load a real chunk
//    again, so every LDS byte an operand read touches holds input data.
#pragma once

#include "attn_device.h"
#include "kernels.h"

namespace sdpa {

template <int D, int DV>
struct FastCfg {
  static constexpr int MF = 32, KW = 16, ACC = 16, KG = 2;
  static constexpr int QB = 1;                  // 32-row query blocks per wavefront
  static constexpr int ROWS = QB * MF;          // query rows per wavefront
  static constexpr int BN = 32;                 // keys per tile
  static constexpr int NW = 4;                  // wavefronts per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int LW = D <= 64 && DV <= 64 ? 64 : 128;  // LDS row width (elements)
  static constexpr int RB = LW * 2;             // bytes per LDS row
  static constexpr int CPR = LW / 8;            // 16-byte chunks per LDS row
  static constexpr int KCH = D / 8, VCH = DV / 8;  // real chunks of a K and a V row
  static constexpr int ROWS_PER_KB = 1024 / RB; // rows filled by one direct-load instruction
  static constexpr int TILE_BYTES = BN * RB;    // one K or V tile
  static constexpr int LOADS = TILE_BYTES / 1024;  // direct-load instructions per tile and tensor
  static constexpr int LOADS_PER_WAVE = LOADS / NW;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K then V
  static constexpr int LOADS_PER_TILE = 2 * LOADS_PER_WAVE;  // per wavefront, K and V
  static constexpr int NQC = D / KW;            // k-steps of QK^T
  static constexpr int NSB = BN / MF;           // 32-key blocks per tile
  static constexpr int NPV = BN / KW;           // k-steps of PV
  static constexpr int NDB = (DV + MF - 1) / MF;  // 32-column output blocks
  static constexpr int NPK = NSB * ACC / 2;     // packed weight pairs per query block
  static constexpr int WPE = 3;                 // wavefronts per SIMD the registers allow
  static constexpr int STAGES = 3;              // LDS ring of K/V tiles
  static_assert((D == DV && (D == 64 || D == 80 || D == 96 || D == 128)) || (D == 96 && DV == 64),
                "the pipelined prefill covers (64,64), (80,80), (96,96), (128,128) and (96,64)");
  static_assert(D % KW == 0 && DV % 8 == 0, "whole k-steps and 8-column store groups");
  static_assert(LOADS % NW == 0, "loads divide among wavefronts");
};

// chunk permutations (XOR masks) for the K and V tiles of an LW-wide LDS layout
template <int LW> __device__ __forceinline__ int swz_k(int row) { return row % (LW / 8); }
// (V: the row's place among the rows sharing one 256-byte line of banks;
// rows of 256 bytes or more start on the same bank, so consecutive rows differ)
template <int LW> __device__ __forceinline__ int swz_v(int row) {
  constexpr int RPL = LW * 2 >= 256 ? 1 : 256 / (LW * 2);  // rows per 256-byte line
  constexpr int NX = LW / 32 < 4 ? LW / 32 : 4;
  return 4 * ((row / RPL) % NX);
}
// the chunk a lane loads into layout slot `slot` of a row with `real` chunks:
// slots past the real ones take a real chunk again
template <int CPR, int REAL> __device__ __forceinline__ int fast_src_chunk(int slot) {
  if constexpr (REAL < CPR) return slot < REAL ? slot : slot - REAL;
  return slot;
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and leaves the other counters alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8). Given as the builtin so that
// the compiler's own wait tracking sees it.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// BOOLMASK: the call has a boolean mask (packed into bits); the other
// instantiation serves causal and unmasked calls without the mask-word code.
template <class E, int D, int DV, bool BOOLMASK>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FastCfg<D, DV>::WPE, FastCfg<D, DV>::WPE)))
prefill_fast_kernel(FwdArgs a) {
  using C = FastCfg<D, DV>;
  constexpr int MF = C::MF, ACC = C::ACC, BN = C::BN, QB = C::QB;
  using acc_t = f32x16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps control flow scalar
  const int col = lane % MF;
  const int kg = lane / MF;

  const int heads = a.Hq * a.B / a.head_blocks;
  const int wph = C::NW / heads;
  const int bm = wph * C::ROWS;
  int hb, qb;
  prefill_item((int)blockIdx.x, a.head_blocks, a.nqb, a.group / heads, hb, qb);
  const int groups_per_b = a.Hq / heads;
  const int b = hb / groups_per_b;
  const int h0 = (hb % groups_per_b) * heads;
  const int hkv = h0 / a.group;
  const int h = h0 + w / wph;
  const int wi0 = qb * bm + (w % wph) * C::ROWS;
  const int shift = a.Lk - a.Lq;

  // keys the workgroup needs: up to its last row's causal limit and, with a
  // sliding window, from its first row's window start; it visits tiles
  // tb .. tb + ntiles - 1
  int kend = a.Lk;
  if (a.mask_kind == kMaskCausal) kend = min(a.Lk, min(qb * bm + bm, a.Lq) - 1 + shift + 1);
  if (kend < 0) kend = 0;
  int kbeg = 0;
  if (a.window > 0) kbeg = min(max(0, qb * bm + shift - a.window + 1), kend);
  const int tb = kbeg / BN;
  const int ntiles = max((kend + BN - 1) / BN - tb, 0);
  // keys every row of this wavefront sees: [w_klo, w_kfull)
  int w_kfull = BOOLMASK ? 0 : a.Lk;
  if (a.mask_kind == kMaskCausal) w_kfull = min(a.Lk, wi0 + shift + 1);
  int w_klo = 0;
  if (a.window > 0) w_klo = min(wi0 + C::ROWS, a.Lq) - 1 + shift - a.window + 1;
  const bool wave_live = wi0 < a.Lq;

  int iq[QB];
  u32x4 qop[QB][C::NQC];
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    iq[r] = wi0 + r * MF + col;
    const uint16_t* qp = (const uint16_t*)a.q + b * a.qs[0] + h * a.qs[1] + (int64_t)iq[r] * a.qs[2];
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (iq[r] < a.Lq) x = ld_global16(qp + c * C::KW + kg * 8);
      qop[r][c] = x ^ a.qsign;
    }
  }

  // boolean mask: each lane's row of packed mask words; the word of tile t
  // is fetched one step ahead (before that step's tile loads are issued)
  constexpr bool bool_mask = BOOLMASK;
  const uint32_t* mbrow[QB];
  uint32_t mw_cur[QB], mw_nxt[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    mbrow[r] = bool_mask ? a.mbits + (size_t)min(iq[r], a.Lq - 1) * a.mwords : nullptr;
    mw_cur[r] = 0u;
    mw_nxt[r] = (bool_mask && ntiles > 0) ? mbrow[r][tb] : 0u;
  }

  acc_t o[QB][C::NDB];
#pragma unroll
  for (int r = 0; r < QB; ++r)
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) o[r][d] = acc_t{};
  float m[QB], l[QB], tmax[QB];
  float sink2 = 0.0f;
  const bool has_sink = a.sinks != nullptr;
  if (has_sink) sink2 = half_to_f32<E>(((const uint16_t*)a.sinks)[h]) * kLog2e;
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    m[r] = has_sink ? sink2 : -INFINITY;
    l[r] = 0.0f;
    tmax[r] = -INFINITY;
  }

  // K/V rows through their element strides (row strides below 2^26 bytes, so
  // the per-lane offsets within a tile fit in 32 bits)
  const uint8_t* kbase = (const uint8_t*)a.k + (b * a.ks[0] + hkv * a.ks[1]) * 2;
  const uint8_t* vbase = (const uint8_t*)a.v + (b * a.vs[0] + hkv * a.vs[1]) * 2;
  const uint32_t krs = (uint32_t)(a.ks[2] * 2), vrs = (uint32_t)(a.vs[2] * 2);

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
    offk[it] = row * krs + fast_src_chunk<C::CPR, C::KCH>(ld_slot ^ swz_k<C::LW>(row)) * 16;
    offv[it] = row * vrs + fast_src_chunk<C::CPR, C::VCH>(ld_slot ^ swz_v<C::LW>(row)) * 16;
  }
  auto issue_tile = [&](int k0, uint8_t* sbase) {
    const uint8_t* kt = kbase + (size_t)k0 * krs;
    const uint8_t* vt = vbase + (size_t)k0 * vrs;
    const bool tail = k0 + BN > a.Lk;
#pragma unroll
    for (int it = 0; it < C::LOADS_PER_WAVE; ++it) {
      uint32_t ok = offk[it], ov = offv[it];
      if (tail) {
        // rows past the end read the last real row instead; those keys get
        // weight 0. Tiles are issued only below the workgroup's kend <= Lk, so
        // k0 <= Lk - 1 and the offset, (Lk - 1 - k0) rows plus the chunk,
        // stays non-negative in this unsigned arithmetic.
        const uint32_t over = (uint32_t)max(k0 + ldrow[it] - (a.Lk - 1), 0);
        ok -= over * krs;
        ov -= over * vrs;
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

  // per-lane byte offsets of the K and V^T operands within a stage, fixed for the
  // whole walk: each LDS read is then one lane register plus the stage's
  // constant offset (folded into the instruction), with no address arithmetic
  uint32_t ko[C::NQC][C::NSB];
#pragma unroll
  for (int c = 0; c < C::NQC; ++c)
#pragma unroll
    for (int nb = 0; nb < C::NSB; ++nb) {
      const int row = nb * MF + col;
      ko[c][nb] = row * C::RB + (((2 * c + kg) ^ swz_k<C::LW>(row)) * 16);
    }
  // V^T operands: the providers of every read sit on key rows vk0 + kofs, with
  // kofs a multiple of 8 fixed per read; the V swizzle depends on the row only
  // through its residue mod 4 (two rows per 256 bytes at 64-wide heads: mod 4
  // of row / 2), which kofs leaves unchanged. So each 32-column block takes one
  // lane offset, and kofs * RB folds into the instruction's offset field.
  const int vk0 = acc_row<MF>(0, kg) + tr_e;
  uint32_t vb[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
    vb[db] = C::TILE_BYTES + vk0 * C::RB + tr_half + (((db * 4 + tr_chunk) ^ swz_v<C::LW>(vk0)) * 16);

  // S^T = K Q^T for one tile into s (zeroed here)
  auto qk = [&](const uint8_t* Ks, acc_t (&s)[QB][C::NSB]) {
#pragma unroll
    for (int r = 0; r < QB; ++r)
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb) s[r][nb] = acc_t{};
#pragma unroll
    for (int c = 0; c < C::NQC; ++c)
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(Ks + ko[c][nb]);
#pragma unroll
        for (int r = 0; r < QB; ++r) s[r][nb] = mma16<E, MF>(kop, qop[r][c], s[r][nb]);
      }
  };

  // scaled row maxima of a tile every row sees in full
  auto tile_max_full = [&](acc_t (&s)[QB][C::NSB]) {
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) mx = fmaxf(mx, s[r][nb][i]);
      mx = row_max<MF>(mx);
      tmax[r] = mx * a.c;
    }
  };
  // the same for a tile some row does not fully see: hidden scores become -inf
  auto tile_max_masked = [&](int t, acc_t (&s)[QB][C::NSB], const uint32_t (&mw)[QB]) {
    const int k0 = t * BN;
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      const bool row_ok = iq[r] < a.Lq;
      if constexpr (BOOLMASK) {
        // the tile's 32 keys are one word of the row's packed mask (zero past
        // Lk); the lane's keys sit at acc_row(i, kg) = acc_row(i, 0) + 4 kg
        static_assert(BN == 32 && C::NSB == 1, "one mask word per tile");
        const uint32_t wsh = row_ok ? (mw[r] >> (4 * kg)) : 0u;
#pragma unroll
        for (int i = 0; i < ACC; ++i) s[r][0][i] = keep_if_bit(s[r][0][i], wsh, acc_row<MF>(i, 0));
      } else {
        // causal (or no mask past the last key)
        // causal (and window) limits, or no mask past the last key
        const int lim = a.mask_kind == kMaskCausal ? min(iq[r] + shift, a.Lk - 1) : a.Lk - 1;
        const int lo = a.window > 0 ? iq[r] + shift - a.window : -1;
#pragma unroll
        for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
          for (int i = 0; i < ACC; ++i) {
            const int key = k0 + nb * MF + acc_row<MF>(i, kg);
            const bool vis = row_ok & (key <= lim) & (key > lo);
            s[r][nb][i] = vis ? s[r][nb][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; ++i) mx = fmaxf(mx, s[r][nb][i]);
      mx = row_max<MF>(mx);
      tmax[r] = (mx == -INFINITY) ? -INFINITY : mx * a.c;
    }
  };

  // weights of one tile, rounded to 16 bits for the MFMA; the running sum adds
  // the same rounded weights (two per v_dot2), so numerator and denominator agree
  auto weights = [&](acc_t (&s)[QB][C::NSB], uint32_t (&pk)[QB][C::NPK]) {
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      const float mu = (m[r] == -INFINITY) ? 0.0f : m[r];
#pragma unroll
      for (int nb = 0; nb < C::NSB; ++nb)
#pragma unroll
        for (int i = 0; i < ACC; i += 2) {
          const float p0 = fast_exp2(fmaf(s[r][nb][i], a.c, -mu));
          const float p1 = fast_exp2(fmaf(s[r][nb][i + 1], a.c, -mu));
          pk[r][(nb * ACC + i) / 2] = pack2<E>(p0, p1);
        }
      float lsum0 = 0.0f, lsum1 = 0.0f;
#pragma unroll
      for (int j = 0; j < C::NPK; j += 2) {
        lsum0 = pair_sum<E>(pk[r][j], lsum0);
        lsum1 = pair_sum<E>(pk[r][j + 1], lsum1);
      }
      l[r] += lsum0 + lsum1;
    }
  };

  // O^T += V^T P^T for one tile (St: the tile's stage; V follows K in it)
  auto pv = [&](const uint8_t* St, const uint32_t (&pk)[QB][C::NPK]) {
#pragma unroll
    for (int t8 = 0; t8 < C::NPV; ++t8) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int kA = ((8 * t8) / ACC) * MF + acc_row<MF>((8 * t8) % ACC, 0);
        const int kB = ((8 * t8 + 4) / ACC) * MF + acc_row<MF>((8 * t8 + 4) % ACC, 0);
        const u32x2 ra = lds_read_tr16((const uint16_t*)(St + vb[db] + kA * C::RB));
        const u32x2 rb = lds_read_tr16((const uint16_t*)(St + vb[db] + kB * C::RB));
        const u32x4 va = {ra[0], ra[1], rb[0], rb[1]};
#pragma unroll
        for (int r = 0; r < QB; ++r) {
          const u32x4 pb = {pk[r][4 * t8], pk[r][4 * t8 + 1], pk[r][4 * t8 + 2], pk[r][4 * t8 + 3]};
          o[r][db] = mma16<E, MF>(va, pb, o[r][db]);
        }
      }
    }
  };

  // Pipelined step t: tile t's weights and PV, tile t+1's scores and maxima.
  // Scur holds tile t, Snext tile t+1 and Sload (last read for tile t-1)
  // receives tile t + STAGES - 1.
  acc_t sa[QB][C::NSB], sb[QB][C::NSB];
  uint32_t pk[QB][C::NPK];
  auto step = [&](int t, acc_t (&scur)[QB][C::NSB], acc_t (&snext)[QB][C::NSB], const uint8_t* Scur,
                  const uint8_t* Snext, uint8_t* Sload) {
    if constexpr (BOOLMASK) {
#pragma unroll
      for (int r = 0; r < QB; ++r) {
        mw_cur[r] = mw_nxt[r];
        mw_nxt[r] = t + 1 < ntiles ? mbrow[r][tb + t + 1] : 0u;
      }
    }
    // Tile t+1 has landed: its loads are the only ones outstanding. The
    // barrier then also guarantees every wavefront has finished tile t-1 (its
    // LDS reads are drained before it arrives), whose stage the next issue
    // refills. A plain s_barrier: the release fence of __syncthreads would
    // also wait for the vector-memory counter.
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + C::STAGES - 1 < ntiles) issue_tile((tb + t + C::STAGES - 1) * BN, Sload);
    const int kt = tb + t;  // key tile
    if ((kt + 1) * BN > w_kfull || kt * BN < w_klo) tile_max_masked(kt, scur, mw_cur);
#pragma unroll
    for (int r = 0; r < QB; ++r) softmax_rebase<C::NDB>(tmax[r], m[r], l[r], o[r]);
    qk(Snext, snext);
    weights(scur, pk);
    pv(Scur, pk);
    tile_max_full(snext);
  };

  // prologue: tiles 0 .. STAGES-2 in flight, tile 0's scores and maxima
  if (ntiles > 0) issue_tile(tb * BN, lds0);
  if (ntiles > 1) issue_tile((tb + 1) * BN, lds1);
  if (ntiles > 1) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(C::LOADS_PER_TILE));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ntiles > 0) {
    qk(lds0, sa);
    tile_max_full(sa);
  }
  // Stage of step t is t % STAGES and scores alternate between sa (even t)
  // and sb, so the loop is unrolled by lcm(STAGES, 2) and every call has fixed
  // arguments. The last step also scores a next tile, from a stage holding
  // stale data, and discards the result: one extra QK^T per workgroup keeps a
  // separate final step out of the loop.
  for (int t = 0; t < ntiles; t += 6) {
    step(t, sa, sb, lds0, lds1, lds2);
    if (t + 1 >= ntiles) break;
    step(t + 1, sb, sa, lds1, lds2, lds0);
    if (t + 2 >= ntiles) break;
    step(t + 2, sa, sb, lds2, lds0, lds1);
    if (t + 3 >= ntiles) break;
    step(t + 3, sb, sa, lds0, lds1, lds2);
    if (t + 4 >= ntiles) break;
    step(t + 4, sa, sb, lds1, lds2, lds0);
    if (t + 5 >= ntiles) break;
    step(t + 5, sb, sa, lds2, lds0, lds1);
  }

  if (!wave_live) return;
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    float lt = row_sum<MF>(l[r]);
    if (has_sink) lt += fast_exp2(sink2 - m[r]);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (iq[r] >= a.Lq) continue;
    uint16_t* op = (uint16_t*)a.out + ((size_t)(b * a.Hq + h) * a.Lq + iq[r]) * DV;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < ACC / 4; ++g4) {
        if (db * MF + g4 * 4 * C::KG >= DV) continue;   // spare columns of the last block
        const int dv = db * MF + g4 * 4 * C::KG + kg * 4;
        const u32x2 st = {pack2<E>(o[r][db][g4 * 4 + 0] * inv, o[r][db][g4 * 4 + 1] * inv),
                          pack2<E>(o[r][db][g4 * 4 + 2] * inv, o[r][db][g4 * 4 + 3] * inv)};
        st_global8(op + dv, st);
      }
  }
}

}  // namespace sdpa
