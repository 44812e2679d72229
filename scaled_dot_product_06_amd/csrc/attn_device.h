// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers and their lane layouts, LDS transpose reads, cross-lane row
// reductions and the online-softmax state update.
//
// The online-softmax recurrence follows lattice-inference
// "src/attention/flash.rs" (run_tiled_attention_head): per key tile, a new row
// maximum, a rescale factor for the running sum and output, tile weights, and
// a final division by the running sum (zero rows when it is zero). Masked keys
// carry no weight at all. Here the arithmetic is base 2 (scores are multiplied
// by scale*log2(e) and exponentiated with exp2), which is the same softmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// A row's reference maximum is moved only when a tile's maximum exceeds it by
// more than this many powers of two, so most tiles skip the output rescale.
// Softmax is invariant to the reference, and weights stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

struct ElemBF16 {};
struct ElemF16 {};

// ---- MFMA tile traits ------------------------------------------------------
// MF x MF output tile; every lane holds 8 consecutive k-elements of A and B.
// Lane l: column/row index l % MF, k-group l / MF (KG groups of 8 k's).
// Accumulator element i of lane l sits at row acc_row(i, l / MF), column l % MF.
template <int MF> struct Mfma;
template <> struct Mfma<32> {
  static constexpr int KW = 16;   // k per instruction (16-bit inputs)
  static constexpr int ACC = 16;  // accumulators per lane
  static constexpr int KG = 2;
  static constexpr int KWF = 2;   // k per instruction for f32 inputs
  typedef f32x16 acc_t;
};
template <> struct Mfma<16> {
  static constexpr int KW = 32;
  static constexpr int ACC = 4;
  static constexpr int KG = 4;
  static constexpr int KWF = 4;
  typedef f32x4 acc_t;
};

template <int MF>
__device__ __forceinline__ constexpr int acc_row(int i, int kg) {
  return (i / 4) * (4 * Mfma<MF>::KG) + kg * 4 + (i % 4);
}

template <class E, int MF>
__device__ __forceinline__ typename Mfma<MF>::acc_t mma16(u32x4 a, u32x4 b, typename Mfma<MF>::acc_t c);

template <> __device__ __forceinline__ f32x16 mma16<ElemBF16, 32>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mma16<ElemF16, 32>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma16<ElemBF16, 16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma16<ElemF16, 16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int MF>
__device__ __forceinline__ typename Mfma<MF>::acc_t mma_f32(float a, float b, typename Mfma<MF>::acc_t c);
template <> __device__ __forceinline__ f32x16 mma_f32<32>(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma_f32<16>(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- 16-bit element helpers -------------------------------------------------
template <class E> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<ElemBF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<ElemF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
template <class E> __device__ __forceinline__ float half_to_f32(uint16_t h);
template <> __device__ __forceinline__ float half_to_f32<ElemBF16>(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
template <> __device__ __forceinline__ float half_to_f32<ElemF16>(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
template <class E> __device__ __forceinline__ uint16_t f32_to_half(float x) {
  return (uint16_t)(pack2<E>(x, 0.0f) & 0xFFFFu);
}

// acc + lo + hi of a packed pair of 16-bit values (one v_dot2 against (1, 1)).
template <class E> __device__ __forceinline__ float pair_sum(uint32_t packed, float acc);
template <> __device__ __forceinline__ float pair_sum<ElemBF16>(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}
template <> __device__ __forceinline__ float pair_sum<ElemF16>(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
}

// ---- memory helpers ----------------------------------------------------------
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming (non-temporal) 16-byte load, for data read exactly once.
__device__ __forceinline__ u32x4 ld_global16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_global8(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

#define SDPA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))


// Transposed 4 x 16-bit LDS read (gfx950 ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane j receives element (j % 4) of the 8-byte chunks that
// lanes 4e + j/4 (e = 0..3) point at, in element order e.  If provider lane
// 4e + c points at row (r0 + e), column (c0 + 4c) of a row-major 16-bit
// matrix, lane j receives rows r0..r0+3 of column c0 + j.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SDPA_LDS(i16x4, p));
  return __builtin_bit_cast(u32x2, r);
}

// ---- cross-lane reductions over the lanes that hold one row ---------------------
// permlane32_swap(x, x) returns {x[l], x[l-32]} above lane 31 and {x[l], x[l+32]}
// (as {first, second} = {x[l] or x[l-32], x[l+32] or x[l]}) so the pair holds
// both halves' values in every lane.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int MF> __device__ __forceinline__ float row_max(float x) {
  x = max_xor32(x);
  if constexpr (MF == 16) x = fmaxf(x, __shfl_xor(x, 16));
  return x;
}
template <int MF> __device__ __forceinline__ float row_sum(float x) {
  x = sum_xor32(x);
  if constexpr (MF == 16) x = x + __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x if bit `pos` of `word` is set, else -inf: a signed one-bit field extract
// gives an all-ones or all-zeros keep mask, and one bitfield insert selects.
__device__ __forceinline__ float keep_if_bit(float x, uint32_t word, int pos) {
  const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)word, (unsigned)pos, 1u);
  return __uint_as_float((keep & __float_as_uint(x)) | (~keep & 0xFF800000u));
}

// Additive masks: four consecutive values (keys key .. key+3) of one mask row,
// fetched with one 8-byte (16-bit types) or 16-byte (f32) load. The row needs
// only element alignment: global memory is accessed in unaligned mode, where
// multi-dword loads take any byte address. The last group of a row, which may
// run past Lk, is read element by element.
//
// 16-bit types: the raw patterns (two per word), so a prefetched tile of the
// mask takes half the registers; keys at or past Lk hold the pattern of -inf.
template <class E> __device__ __forceinline__ uint16_t neg_inf_bits();
template <> __device__ __forceinline__ uint16_t neg_inf_bits<ElemBF16>() { return 0xFF80u; }
template <> __device__ __forceinline__ uint16_t neg_inf_bits<ElemF16>() { return 0xFC00u; }
template <class E> __device__ __forceinline__ u32x2 mask4_bits(const void* row, int key, int Lk) {
  const uint16_t* p = (const uint16_t*)row + key;
  if (key + 4 <= Lk) {
    u32x2 x;
    __builtin_memcpy(&x, p, 8);
    return x;
  }
  uint32_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = key + e < Lk ? p[e] : neg_inf_bits<E>();
  return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}
// Element e (0..3) of a mask4_bits group, widened and converted to base 2.
template <class E> __device__ __forceinline__ float mask_bits_value(u32x2 g, int e) {
  const uint32_t w = g[e / 2];
  return half_to_f32<E>((uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu))) * kLog2e;
}

// f32: the values converted to base 2 (times log2 e); keys at or past Lk read as -inf.
__device__ __forceinline__ f32x4 mask4_f32(const void* row, int key, int Lk) {
  const float* p = (const float*)row + key;
  f32x4 r;
  if (key + 4 <= Lk) {
    __builtin_memcpy(&r, p, 16);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = key + e < Lk ? p[e] : -INFINITY;
  }
  return r * kLog2e;
}

// Work item (head block hb, query block qb) of prefill workgroup n, for a 1-D
// grid of head_blocks * nqb workgroups. The dispatcher deals workgroups to the
// 8 XCDs round-robin; this order makes each XCD walk the head blocks of one
// (batch, kv head) pair at a time, longest (latest) query blocks first, so the
// pair's K/V stays resident in that XCD's L2.
constexpr int kXcds = 8;
__device__ __forceinline__ void prefill_item(int n, int head_blocks, int nqb, int hb_per_pair, int& hb, int& qb) {
  const int pairs = head_blocks / hb_per_pair;
  const int per_pair = hb_per_pair * nqb;
  int pair, r;
  if (pairs % kXcds == 0) {
    const int xcd = n % kXcds, s = n / kXcds;
    pair = (s / per_pair) * kXcds + xcd;
    r = s % per_pair;
  } else {
    pair = n / per_pair;
    r = n % per_pair;
  }
  qb = nqb - 1 - r / hb_per_pair;
  hb = pair * hb_per_pair + r % hb_per_pair;
}

// Online-softmax reference update for one wave. `tile_max` is the row's
// largest scaled score in the new tile (-inf if it sees none). When any row's
// tile maximum passes its reference by more than kRescaleSlack, every row moves
// its reference to max(old, tile) and rescales its running sum and output.
template <int NACC, class Acc>
__device__ __forceinline__ void softmax_rebase(float tile_max, float& m, float& l, Acc* o) {
  const bool need = tile_max > m + kRescaleSlack;
  if (__any(need)) {
    const float m_new = fmaxf(m, tile_max);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < NACC; ++d) o[d] *= alpha;
    m = m_new;
  }
}

}  // namespace sdpa
