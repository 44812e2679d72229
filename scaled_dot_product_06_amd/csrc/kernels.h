// Kernel argument block and the launcher entry points the host router calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

enum Elem { kF32 = 0, kF16 = 1, kBF16 = 2 };
enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskBool = 2, kMaskAdditive = 3 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const uint8_t* mask;   // [Lq, Lk] bytes when mask_kind == kMaskBool
  const uint32_t* mbits; // 16-bit prefill with a boolean mask: the mask packed as
                         // [Lq, mwords] words, bit j of word w = key 32w + j visible
  int mwords;            // ceil(Lk / 32)
  const void* sinks;     // [Hq] in the element type, or null
  // element strides (batch, head, row) of q, k and v; the feature axis is contiguous
  int64_t qs[3], ks[3], vs[3];
  // additive mask (mask_kind == kMaskAdditive): values in the element type at
  // amask + b*ms[0] + h*ms[1] + i*ms[2] + j, added to the scaled scores
  const void* amask;
  int64_t ms[3];
  int B, Hq, Hkv, Lq, Lk;
  int group;             // Hq / Hkv
  int mask_kind;
  int window;            // causal sliding window: row i (position pos = i + Lk - Lq) reads keys
                         // pos - window < j <= pos; 0 for none
  int koff;              // decode: first key the windowed rows read (0 without a window)
  // paged caches: k and v are [blocks, Hkv, bs, D/Dv]; sequence b's key j is row j % bs
  // of block table[b][j / bs]; its length is lengths[b] (both clamped in the kernel)
  const int32_t* table;  // [B, max_blocks]
  const int32_t* lengths;  // [B]
  int blocks, bs, max_blocks;
  float c;               // |scale| * log2(e): scores are taken as c * q.k in base 2
  uint32_t qsign;        // XOR applied to q bits (flips q's sign when scale < 0)
  // prefill
  int nqb;               // query blocks per head
  int head_blocks;       // B * Hq / heads_per_group
  // decode
  int rows;              // group * Lq: query rows packed into one wavefront
  int kps;               // keys per split (one wavefront's key range)
  int nsplit;            // splits per (batch, kv head)
  float* part;           // scratch: per split and row, {m, l} then Dv floats of output
};

// Geometry chosen by the host for a prefill launch.
struct PrefillShape {
  int mf;         // MFMA tile (rows per wave): 32 or 16
  int waves;      // waves per workgroup
  int heads;      // query heads per workgroup (share the K/V tiles)
  int block_n;    // keys per tile
  int block_m;    // query rows per head per workgroup
  int ksplit;     // > 1: the workgroup's waves split the keys of one query block
};

struct DecodeShape {
  int mf;         // 16 or 32 (>= group * Lq)
  int waves;      // waves (splits) per workgroup
  int block_n;    // keys per tile
};

// Each launcher returns hipSuccess or the launch error; `ok` is false when no
// kernel is built for the (dtype, D, Dv) combination.
hipError_t launch_prefill(int elem, int D, int Dv, const PrefillShape& s, const FwdArgs& a,
                          hipStream_t stream, bool* ok);
hipError_t launch_decode(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a,
                         hipStream_t stream, bool* ok);
hipError_t launch_prefill_f32_paged(int D, int Dv, const PrefillShape& s, const FwdArgs& a, hipStream_t stream,
                                    bool* ok);
hipError_t launch_decode_paged(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a,
                               hipStream_t stream, bool* ok);
hipError_t launch_paged_write(void* cache, const void* rows, const int32_t* slots, int64_t n, int64_t blocks,
                              int64_t Hkv, int64_t bs, int64_t row_bytes, hipStream_t stream);
hipError_t launch_zero_fill(void* out, int64_t bytes, hipStream_t stream);
hipError_t launch_mask_bits(const uint8_t* mask, uint32_t* bits, int64_t Lq, int64_t Lk, hipStream_t stream);
constexpr int64_t mask_words(int64_t Lk) { return (Lk + 31) / 32; }
// The pipelined and generic 16-bit prefill kernels read a boolean mask as packed
// bits, made by a first small kernel; the key-split kernel reads the bytes.
constexpr bool prefill_packs_mask(int elem, int mask_kind) { return elem != kF32 && mask_kind == kMaskBool; }

// Geometry rules shared by the launchers (template arguments) and the planner.
constexpr int kPrefillWaves = 4;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeBN = 32;       // keys per decode tile
// value columns per decode-reduce workgroup: 32 when they divide Dv, else 16
constexpr int reduce_cols(int DV) { return DV % 32 == 0 ? 32 : 16; }
constexpr int head_max(int D, int Dv) { return D > Dv ? D : Dv; }
// The 16-bit prefill shapes with heads up to 128 wide, (64,64), (80,80), (96,96),
// (128,128) and (96,64), run the pipelined direct-load kernel (32-row tiles,
// 32-key steps), except with an additive mask (the generic kernel reads it).
constexpr bool prefill_can_fast(int elem, int D, int Dv, int mask_kind) {
  return elem != kF32 && mask_kind != kMaskAdditive &&
         ((D == Dv && (D == 64 || D == 80 || D == 96 || D == 128)) || (D == 96 && Dv == 64));
}
constexpr int kFastRows = 32, kFastBN = 32;
// The key-split kernel: 16-row tiles, and the workgroup's wavefronts in two key
// lanes that each take 32 keys of every 64-key step, so each SIMD holds two
// wavefronts. 16-bit heads of 192 columns or more, (192,192), (192,128) and
// (256,256), run it on every grid and with every mask (a 32-row tile of these
// heads leaves room for one wavefront per SIMD), and so do 128-wide heads with an
// additive mask;
// narrower heads ((64,64), (80,80), (96,96), (128,128), (96,64)) run it when the
// pipelined kernel's grid for one batch item would have fewer than
// kKsplitSmallGrid workgroups: at one workgroup per compute unit or less, the
// twice as many 16-row workgroups and the halved key chain of each win; on
// fuller grids the 32-row pipelined tiles do. The rule leaves the batch size out,
// so a batch item takes the same kernel, and gives the same bits, alone or
// within a batch.
constexpr int kKsplitLanes = 2, kKsplitRows = 16, kKsplitBN = 32;
constexpr int kKsplitSmallGrid = 256;
constexpr bool prefill_can_ksplit(int elem, int D, int Dv) {
  return elem != kF32 && ((D == Dv && (D == 64 || D == 80 || D == 96 || D == 128 || D == 192 || D == 256)) ||
                          (D == 96 && Dv == 64) || (D == 192 && Dv == 128));
}
// Calls that take it on every grid: heads of 192 columns or more, and 128-wide
// heads with an additive mask (the pipelined kernel reads none, and the generic
// kernel measured slower on every grid).
constexpr bool prefill_ksplit_always(int D, int Dv, int mask_kind) {
  return (D >= 192 && Dv >= 128) || (D == 128 && Dv == 128 && mask_kind == kMaskAdditive);
}
// Generic kernel: 32x32 MFMA tiles (32 query rows per wavefront) up to
// 128-wide heads; 16x16 tiles above, where a 32-row output accumulator would
// leave too few registers for its staging.
constexpr int prefill_generic_mf(int elem, int D, int Dv) { return head_max(D, Dv) <= 128 ? 32 : 16; }
// f32 calls whose 32-row grid (for one batch item, so that a batch item gets
// the same tiles alone or in a batch) has fewer workgroups than this take
// 16-row tiles instead: twice the wavefronts, each with half the rows.
constexpr int kF32SmallGrid = 256;
// Those calls (unless they carry an additive mask) run the key-split f32
// kernel: one 16-row query block per workgroup, its keys split among the
// workgroup's waves in tiles of this many keys.
constexpr int f32_split_bn(int D, int Dv) { return head_max(D, Dv) <= 64 ? 32 : 16; }
constexpr int prefill_generic_bn(int elem, int D, int Dv) {
  return elem == kF32 ? (head_max(D, Dv) <= 128 ? 32 : 16) : (head_max(D, Dv) > 256 ? 32 : 64);
}
constexpr int prefill_waves(int elem, int D, int Dv) { return kPrefillWaves; }
// 16x16 tiles when the packed query rows fit (and the head is a whole number
// of 32-wide k-steps), else 32x32.
constexpr int decode_mf(int D, int rows) { return rows <= 16 && D % 32 == 0 ? 16 : 32; }

// The (D, Dv) pairs kernels are built for.
#define SDPA_HEAD_PAIRS(X) \
  X(64, 64) X(80, 80) X(96, 96) X(128, 128) X(192, 192) X(256, 256) X(512, 512) X(96, 64) X(192, 128)

inline bool head_pair_supported(long long D, long long Dv) {
#define SDPA_CHECK_PAIR(d, dv) if (D == d && Dv == dv) return true;
  SDPA_HEAD_PAIRS(SDPA_CHECK_PAIR)
#undef SDPA_CHECK_PAIR
  return false;
}

}  // namespace sdpa
