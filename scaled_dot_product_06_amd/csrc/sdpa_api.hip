// The C ABI (include/sdpa.h): argument validation, the router between the
// prefill and decode kernels, scratch (decode partials, packed mask bits),
// and the launches.
//
// The router keeps the shape of the rules in nuvec-core
// "tests/attention_plan.rs" (a fused tiled kernel for many queries; for few
// queries a vector kernel split over key partitions in two passes, with more
// partitions as the key count grows), with thresholds set for gfx950: one
// wavefront carries one MFMA tile of query rows, so the decode route applies
// while Lq <= 8 and the (Hq/Hkv) x Lq rows that read one kv head fit in a
// 32-row tile.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/sdpa.h"
#include "kernels.h"

namespace sdpa {

hipError_t launch_prefill_16(int elem, int D, int Dv, const PrefillShape& s, const FwdArgs& a,
                             hipStream_t stream, bool* ok);
hipError_t launch_prefill_f32(int D, int Dv, const PrefillShape& s, const FwdArgs& a, hipStream_t stream,
                              bool* ok);

hipError_t launch_prefill(int elem, int D, int Dv, const PrefillShape& s, const FwdArgs& a,
                          hipStream_t stream, bool* ok) {
  if (elem == kF32) return launch_prefill_f32(D, Dv, s, a, stream, ok);
  return launch_prefill_16(elem, D, Dv, s, a, stream, ok);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) zero_fill_kernel(u32x4_t* out, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    out[i] = u32x4_t{0u, 0u, 0u, 0u};
}

hipError_t launch_zero_fill(void* out, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4_t*)out, n16);
  return hipGetLastError();
}

// Packs the [Lq, Lk] byte mask into bits for the 16-bit prefill kernels: word
// w of row i holds keys 32w..32w+31, bit j set iff mask[i][32w + j] != 0 (keys
// past Lk read as 0). One thread per output word: it reads the word's 32 mask
// bytes with two 16-byte loads (global memory is accessed in unaligned mode,
// so a row may start at any byte) and folds each 4-byte group to 4 bits; the
// last word of a row reads its bytes one by one. A grid-stride loop covers any
// size.
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  // each byte's OR of its bits into the byte's low bit, then the four low bits
  // gathered into bits 24..27 by one multiply (the partial products land on
  // distinct bit positions, so nothing carries)
  uint32_t y = x | (x >> 4);
  y |= y >> 2;
  y |= y >> 1;
  y &= 0x01010101u;
  return (y * 0x01020408u) >> 24;
}

__global__ void __launch_bounds__(256) mask_bits_kernel(const uint8_t* mask, uint32_t* bits, int64_t Lq,
                                                        int64_t Lk, int64_t nwords) {
  const int64_t total = Lq * nwords;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t row = t / nwords, w = t % nwords;
    const uint8_t* p = mask + row * Lk + w * 32;
    uint32_t word = 0u;
    if (w * 32 + 32 <= Lk) {
      u32x4_t lo, hi;
      __builtin_memcpy(&lo, p, 16);
      __builtin_memcpy(&hi, p + 16, 16);
      word = nonzero_bytes4(lo[0]) | (nonzero_bytes4(lo[1]) << 4) | (nonzero_bytes4(lo[2]) << 8) |
             (nonzero_bytes4(lo[3]) << 12) | (nonzero_bytes4(hi[0]) << 16) | (nonzero_bytes4(hi[1]) << 20) |
             (nonzero_bytes4(hi[2]) << 24) | (nonzero_bytes4(hi[3]) << 28);
    } else {
      const int n = (int)(Lk - w * 32);
      for (int j = 0; j < n; ++j) word |= (p[j] != 0 ? 1u : 0u) << j;
    }
    bits[t] = word;
  }
}

hipError_t launch_mask_bits(const uint8_t* mask, uint32_t* bits, int64_t Lq, int64_t Lk, hipStream_t stream) {
  const int64_t words = Lq * mask_words(Lk);
  int64_t blocks = (words + 255) / 256;
  if (blocks > (1 << 16)) blocks = 1 << 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(mask_bits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, bits, Lq, Lk,
                     mask_words(Lk));
  return hipGetLastError();
}

}  // namespace sdpa

using namespace sdpa;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* r) {
  int64_t t;
  if (__builtin_mul_overflow(a, b, &t)) return false;
  return !__builtin_mul_overflow(t, c, r);
}
bool mul4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* r) {
  int64_t t;
  if (!mul3(a, b, c, &t)) return false;
  return !__builtin_mul_overflow(t, d, r);
}

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int64_t pow2_floor(int64_t x) {
  int64_t p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

const int64_t kMaxLen = INT_MAX - 4096;  // positions are 32-bit inside the kernels
const int64_t kMaxGridYZ = 65535;

int elem_size(int dtype) { return dtype == SDPA_F32 ? 4 : 2; }

// First key any query row of a windowed call reads: row i (position
// i + Lk - Lq) reads keys pos - window < j <= pos, so the rows together read
// [Lk - Lq - window + 1, Lk). 0 without a window.
int64_t window_first_key(int64_t Lq, int64_t Lk, int64_t window) {
  if (window <= 0) return 0;
  const int64_t k0 = Lk - Lq - window + 1;
  return k0 > 0 ? k0 : 0;
}

// Keys per decode split for a call whose rows read `nkeys` keys: about a
// 64th of them, a power of two in [64, 1024].
int64_t keys_per_split(int64_t nkeys) {
  int64_t kps = pow2_floor(nkeys / 64 > 0 ? nkeys / 64 : 1);
  if (kps < 64) kps = 64;
  if (kps > 1024) kps = 1024;
  return kps;
}

// Validation shared by the plan and forward entry points; fills `plan` on
// success. `window` is 0 (none) or the windowed calls' window, already
// checked to be >= 1 with a causal mask; a window of at least Lk keys is
// plain causal attention and plans (and runs) as such.
int validate_and_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t Dv,
                      int mask_kind, bool has_mask, bool has_sinks, int dtype, int64_t window,
                      sdpa_plan_t* plan) {
  (void)has_sinks;
  if (B < 0) return fail(SDPA_ERR_INVALID, "B must be >= 0 (got %lld)", (long long)B);
  if (Hq < 0) return fail(SDPA_ERR_INVALID, "Hq must be >= 0 (got %lld)", (long long)Hq);
  if (Hkv < 0) return fail(SDPA_ERR_INVALID, "Hkv must be >= 0 (got %lld)", (long long)Hkv);
  if (Lq < 0) return fail(SDPA_ERR_INVALID, "Lq must be >= 0 (got %lld)", (long long)Lq);
  if (Lk < 0) return fail(SDPA_ERR_INVALID, "Lk must be >= 0 (got %lld)", (long long)Lk);
  if (D < 0) return fail(SDPA_ERR_INVALID, "D must be >= 0 (got %lld)", (long long)D);
  if (Dv < 0) return fail(SDPA_ERR_INVALID, "Dv must be >= 0 (got %lld)", (long long)Dv);
  if (dtype != SDPA_F32 && dtype != SDPA_F16 && dtype != SDPA_BF16)
    return fail(SDPA_ERR_INVALID, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16 (got %d)", dtype);
  if (mask_kind != SDPA_MASK_NONE && mask_kind != SDPA_MASK_CAUSAL && mask_kind != SDPA_MASK_BOOL &&
      mask_kind != SDPA_MASK_ADDITIVE)
    return fail(SDPA_ERR_INVALID, "mask_kind must be 0 (none), 1 (causal), 2 (bool) or 3 (additive) (got %d)",
                mask_kind);
  if (mask_kind == SDPA_MASK_BOOL && !has_mask)
    return fail(SDPA_ERR_INVALID, "mask_kind is SDPA_MASK_BOOL but mask is NULL");
  if (mask_kind == SDPA_MASK_ADDITIVE && !has_mask)
    return fail(SDPA_ERR_INVALID, "mask_kind is SDPA_MASK_ADDITIVE but mask is NULL");
  if (window > 0 && mask_kind != SDPA_MASK_CAUSAL)
    return fail(SDPA_ERR_INVALID, "a window needs mask_kind SDPA_MASK_CAUSAL (got %d)", mask_kind);
  if (Hkv == 0 && Hq != 0) return fail(SDPA_ERR_INVALID, "Hkv must be positive when Hq (%lld) is", (long long)Hq);
  if (Hkv != 0 && Hq % Hkv != 0)
    return fail(SDPA_ERR_INVALID, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  int64_t n;
  const int64_t es = elem_size(dtype);
  if (!mul4(B, Hq, Lq, D, &n) || __builtin_mul_overflow(n, es, &n))
    return fail(SDPA_ERR_INVALID, "shape overflow: B*Hq*Lq*D bytes do not fit in 64 bits");
  if (!mul4(B, Hkv, Lk, D, &n) || __builtin_mul_overflow(n, es, &n))
    return fail(SDPA_ERR_INVALID, "shape overflow: B*Hkv*Lk*D bytes do not fit in 64 bits");
  if (!mul4(B, Hkv, Lk, Dv, &n) || __builtin_mul_overflow(n, es, &n))
    return fail(SDPA_ERR_INVALID, "shape overflow: B*Hkv*Lk*Dv bytes do not fit in 64 bits");
  if (!mul4(B, Hq, Lq, Dv, &n) || __builtin_mul_overflow(n, es, &n))
    return fail(SDPA_ERR_INVALID, "shape overflow: B*Hq*Lq*Dv bytes do not fit in 64 bits");
  if (!mul3(Lq, Lk, 1, &n)) return fail(SDPA_ERR_INVALID, "shape overflow: Lq*Lk mask bytes do not fit in 64 bits");
  if (!head_pair_supported(D, Dv))
    return fail(SDPA_ERR_UNSUPPORTED,
                "head sizes (D=%lld, Dv=%lld) are not built; supported: (64,64) (80,80) (96,96) (128,128) "
                "(192,192) (256,256) (512,512) (96,64) (192,128)",
                (long long)D, (long long)Dv);

  sdpa_plan_t p;
  memset(&p, 0, sizeof p);
  if (B == 0 || Hq == 0 || Lq == 0) {
    p.route = SDPA_ROUTE_EMPTY;
    *plan = p;
    return SDPA_OK;
  }
  if (Lq > kMaxLen) return fail(SDPA_ERR_UNSUPPORTED, "Lq (%lld) exceeds %lld", (long long)Lq, (long long)kMaxLen);
  if (Lk > kMaxLen) return fail(SDPA_ERR_UNSUPPORTED, "Lk (%lld) exceeds %lld", (long long)Lk, (long long)kMaxLen);
  if (B * Hq > INT_MAX) return fail(SDPA_ERR_UNSUPPORTED, "B*Hq (%lld) exceeds INT_MAX", (long long)(B * Hq));
  if (Lk == 0) {
    p.route = SDPA_ROUTE_ZERO_FILL;
    p.kernels = 1;
    int64_t n16 = B * Hq * Lq * Dv * elem_size(dtype) / 16;
    int64_t blocks = (n16 + 255) / 256;
    p.grid[0] = blocks < 1 ? 1 : (blocks > (1 << 20) ? (1 << 20) : blocks);
    p.grid[1] = p.grid[2] = 1;
    *plan = p;
    return SDPA_OK;
  }
  const int64_t group = Hq / Hkv;
  if (dtype != SDPA_F32 && Lq <= 8 && group * Lq <= 32) {
    const int64_t rows = group * Lq;
    // the key partitions follow the keys the rows read (the window's, if any)
    const int64_t nkeys = Lk - window_first_key(Lq, Lk, window);
    const int64_t kps = keys_per_split(nkeys);
    const int64_t nsplit = (nkeys + kps - 1) / kps;
    p.route = SDPA_ROUTE_DECODE;
    p.kernels = 2;
    p.rows_per_wave = decode_mf((int)D, (int)rows);
    p.waves = kDecodeWaves;
    p.block_n = kDecodeBN;
    p.heads_per_group = (int32_t)group;
    p.keys_per_split = kps;
    p.splits = nsplit;
    p.grid[0] = nsplit;
    p.grid[1] = Hkv;
    p.grid[2] = B;
    if (Hkv > kMaxGridYZ || B > kMaxGridYZ || rows > kMaxGridYZ)
      return fail(SDPA_ERR_UNSUPPORTED, "decode grid: Hkv (%lld) and B (%lld) must be <= 65535", (long long)Hkv,
                  (long long)B);
    int64_t sb;
    if (!mul4(B * Hkv, nsplit, rows, (Dv + 4) * 4, &sb))
      return fail(SDPA_ERR_INVALID, "decode scratch size overflows");
    p.scratch_bytes = sb;
    *plan = p;
    return SDPA_OK;
  }
  // the key-split kernel at 16-bit heads of 192 columns or more, 128-wide ones with
  // an additive mask, and narrower ones on small grids; the pipelined kernel
  // (32-row tiles) where it applies; else the generic kernel's geometry
  const int nw = prefill_waves(dtype, (int)D, (int)Dv);
  const int64_t heads = gcd64(group, nw);
  bool kspl = false;
  if (prefill_can_ksplit(dtype, (int)D, (int)Dv)) {
    const int64_t fbm = (nw / heads) * kFastRows;   // a pipelined workgroup's query rows per head
    kspl = prefill_ksplit_always((int)D, (int)Dv, mask_kind) || (Hq / heads) * ((Lq + fbm - 1) / fbm) < kKsplitSmallGrid;
  }
  const bool fast = !kspl && prefill_can_fast(dtype, (int)D, (int)Dv, mask_kind);
  if (kspl) {
    // 16-row query blocks of `heads` heads per workgroup, two key lanes of wavefronts
    const int64_t kbm = (nw / heads) * kKsplitRows;
    const int64_t nqb = (Lq + kbm - 1) / kbm;
    if ((B * Hq / heads) * nqb > INT_MAX)
      return fail(SDPA_ERR_UNSUPPORTED, "Lq (%lld) needs more than INT_MAX workgroups in all", (long long)Lq);
    p.route = SDPA_ROUTE_PREFILL;
    p.kernels = 1;
    p.rows_per_wave = kKsplitRows;
    p.waves = nw * kKsplitLanes;
    p.block_n = kKsplitBN;
    p.heads_per_group = (int32_t)heads;
    p.splits = kKsplitLanes;
    p.grid[0] = (B * Hq / heads) * nqb;
    p.grid[1] = 1;
    p.grid[2] = 1;
    // the kernel reads a boolean mask's bytes itself: one kernel, no scratch
    *plan = p;
    return SDPA_OK;
  }
  int rows = fast ? kFastRows : prefill_generic_mf(dtype, (int)D, (int)Dv);
  bool ksplit = false;
  if (dtype == SDPA_F32 && rows == 32) {
    const int64_t bm32 = (nw / heads) * 32;
    if ((Hq / heads) * ((Lq + bm32 - 1) / bm32) < kF32SmallGrid) {
      rows = 16;
      ksplit = mask_kind != SDPA_MASK_ADDITIVE;
    }
  }
  if (ksplit) {
    // one workgroup per (batch, head, 16-row query block); its waves split the keys
    const int64_t nqb = (Lq + 15) / 16;
    if (B * Hq * nqb > INT_MAX)
      return fail(SDPA_ERR_UNSUPPORTED, "Lq (%lld) needs more than INT_MAX workgroups in all", (long long)Lq);
    p.route = SDPA_ROUTE_PREFILL;
    p.kernels = 1;
    p.rows_per_wave = 16;
    p.waves = nw;
    p.block_n = f32_split_bn((int)D, (int)Dv);
    p.heads_per_group = 1;
    p.splits = nw;
    p.grid[0] = B * Hq * nqb;
    p.grid[1] = 1;
    p.grid[2] = 1;
    *plan = p;
    return SDPA_OK;
  }
  const int64_t bm = (nw / heads) * rows;
  const int64_t nqb = (Lq + bm - 1) / bm;
  if ((B * Hq / heads) * nqb > INT_MAX)
    return fail(SDPA_ERR_UNSUPPORTED, "Lq (%lld) needs %lld query blocks per head block; more than INT_MAX "
                "workgroups in all", (long long)Lq, (long long)nqb);
  p.route = SDPA_ROUTE_PREFILL;
  p.kernels = 1;
  p.rows_per_wave = rows;
  p.waves = nw;
  p.block_n = fast ? kFastBN : prefill_generic_bn(dtype, (int)D, (int)Dv);
  p.heads_per_group = (int32_t)heads;
  p.grid[0] = (B * Hq / heads) * nqb;   // one workgroup per (head block, query block)
  p.grid[1] = 1;
  p.grid[2] = 1;
  if (prefill_packs_mask(dtype, mask_kind)) {
    // the boolean mask is packed into bits by a first small kernel
    int64_t sb;
    if (!mul3(Lq, mask_words(Lk), 4, &sb)) return fail(SDPA_ERR_INVALID, "mask-bit scratch size overflows");
    p.kernels = 2;
    p.scratch_bytes = sb;
  }
  *plan = p;
  return SDPA_OK;
}

// Library scratch (decode partials, packed mask bits): one buffer per device
// and stream, allocated on the stream's first call that needs it and replaced by
// a larger one when a call needs more. A graph captured on the stream keeps the
// address of the buffer it was captured with, so a replaced buffer is kept (on
// the retired list) until sdpa_release_workspace, and a capture never grows the
// buffer: it cannot allocate memory that outlives the graph, and freeing the
// old buffer would pull it from under graphs captured earlier.
struct ScratchEntry {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, ScratchEntry> g_scratch;
std::vector<std::pair<int, void*>> g_retired;  // (device, buffer) replaced by larger ones

// Scratch of at least `bytes` for a call on `stream`: SDPA_OK with *out set, or an
// error code with the message set.
int get_scratch(hipStream_t stream, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  ScratchEntry& s = g_scratch[std::make_pair(dev, stream)];
  if (s.bytes >= bytes) {
    *out = s.ptr;
    return SDPA_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipStreamIsCapturing failed: %s", hipGetErrorString(e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(SDPA_ERR_UNSUPPORTED,
                "the stream is capturing a graph and the call needs %zu bytes of scratch, but the stream holds %zu: "
                "a capture cannot allocate it. Make one call of at least this size (the plan's scratch_bytes) on "
                "the same stream before capturing, or use sdpa_forward_noalloc",
                bytes, s.bytes);
  // at least double, so that a stream's retired buffers hold less than its current one
  size_t want = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
  if (s.ptr && want < 2 * s.bytes) want = 2 * s.bytes;
  void* p = nullptr;
  e = hipMallocAsync(&p, want, stream);
  if (e != hipSuccess)
    return fail(SDPA_ERR_HIP, "scratch allocation of %zu bytes failed: %s", want, hipGetErrorString(e));
  if (s.ptr) g_retired.emplace_back(dev, s.ptr);
  s.ptr = p;
  s.bytes = want;
  *out = p;
  return SDPA_OK;
}

// Allocation-free scratch: one fixed array per device, resident until the
// process ends. In host code the array's name is only a stand-in; the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_fixed_mu;
std::map<int, void*> g_fixed;   // device -> address of its copy of `scratch`

int fixed_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_fixed_mu);
  auto it = g_fixed.find(dev);
  if (it != g_fixed.end()) {
    *out = it->second;
    return SDPA_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(SDPA_ERR_HIP, "hipGetSymbolAddress of the fixed scratch failed on device %d: %s", dev,
                hipGetErrorString(e));
  g_fixed[dev] = ptr;
  *out = ptr;
  return SDPA_OK;
}

// Where a call's scratch comes from: the per-stream cached buffer, or the
// fixed array (allocation-free calls).
enum ScratchSource { kScratchCached = 0, kScratchFixed = 1 };

int call_scratch(int source, hipStream_t stream, size_t bytes, void** out) {
  if (source == kScratchCached) return get_scratch(stream, bytes, out);
  if (bytes > kNoAllocScratchBytes)
    return fail(SDPA_ERR_UNSUPPORTED,
                "the call needs %zu bytes of scratch; sdpa_forward_noalloc holds at most %zu (use sdpa_forward)",
                bytes, kNoAllocScratchBytes);
  return fixed_scratch(out);
}

}  // namespace

extern "C" {

int sdpa_abi_version(void) { return 5; }

const char* sdpa_last_error(void) { return g_err.c_str(); }

int sdpa_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t Dv, int mask_kind,
              int has_mask, int has_sinks, int dtype, sdpa_plan_t* plan) {
  g_err.clear();
  if (!plan) return fail(SDPA_ERR_INVALID, "plan must not be NULL");
  sdpa_plan_t p;
  const int rc = validate_and_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, has_mask != 0, has_sinks != 0, dtype, 0, &p);
  if (rc == SDPA_OK) *plan = p;
  return rc;
}

}  // extern "C"

namespace {

// A windowed call's window as planned: >= 1 (else an error), and 0 (plain
// causal) once it covers every key.
int effective_window(int64_t window, int64_t Lk, int64_t* eff) {
  if (window < 1) return fail(SDPA_ERR_INVALID, "window must be >= 1 (got %lld)", (long long)window);
  if (window > kMaxLen)
    return fail(SDPA_ERR_UNSUPPORTED, "window (%lld) exceeds %lld", (long long)window, (long long)kMaxLen);
  *eff = window >= Lk ? 0 : window;
  return SDPA_OK;
}

// Element strides (batch, head, row) of one [B, H, L, E] operand.
struct Strides {
  int64_t b, h, l;
};
Strides contiguous(int64_t H, int64_t L, int64_t E) { return Strides{H * L * E, L * E, E}; }

// The operands of one forward call as views: data pointers and element strides.
struct Views {
  const void *q, *k, *v;
  Strides qs, ks, vs;
  const void* mask;   // bool: uint8 [Lq, Lk] rows of Lk bytes; additive: dtype elements at ms
  Strides ms;
};

// A view's strides are non-negative and its largest element offset fits in 63 bits.
int check_view(const char* name, const Strides& st, int64_t n0, int64_t n1, int64_t n2, int64_t E) {
  if (st.b < 0 || st.h < 0 || st.l < 0)
    return fail(SDPA_ERR_INVALID, "%s strides must be >= 0 (got %lld, %lld, %lld)", name, (long long)st.b,
                (long long)st.h, (long long)st.l);
  int64_t x, y, z, t;
  if (__builtin_mul_overflow(n0 > 0 ? n0 - 1 : 0, st.b, &x) || __builtin_mul_overflow(n1 > 0 ? n1 - 1 : 0, st.h, &y) ||
      __builtin_mul_overflow(n2 > 0 ? n2 - 1 : 0, st.l, &z) || __builtin_add_overflow(x, y, &t) ||
      __builtin_add_overflow(t, z, &t) || __builtin_add_overflow(t, E, &t) || t > (INT64_MAX >> 2))
    return fail(SDPA_ERR_INVALID, "%s: element offsets overflow", name);
  return SDPA_OK;
}

// 16-byte loads read q, k and v rows: every row start must be 16-byte aligned.
int check_rows_aligned(const char* name, const void* p, const Strides& st, int64_t es) {
  if (((uintptr_t)p & 15) || ((st.b * es) & 15) || ((st.h * es) & 15) || ((st.l * es) & 15))
    return fail(SDPA_ERR_INVALID, "%s must be 16-byte aligned, with every stride * element size a multiple of 16 "
                "bytes", name);
  return SDPA_OK;
}

int forward_impl(const Views& x, void* out, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                 int64_t Dv, float scale, int mask_kind, const void* sinks, int dtype, int64_t window,
                 void* stream_v, int scratch_source = kScratchCached) {
  sdpa_plan_t p;
  int rc = validate_and_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, x.mask != nullptr, sinks != nullptr, dtype,
                             window, &p);
  if (rc != SDPA_OK) return rc;
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  const int64_t es = elem_size(dtype);
  if ((rc = check_view("q", x.qs, B, Hq, Lq, D)) != SDPA_OK) return rc;
  if ((rc = check_view("k", x.ks, B, Hkv, Lk, D)) != SDPA_OK) return rc;
  if ((rc = check_view("v", x.vs, B, Hkv, Lk, Dv)) != SDPA_OK) return rc;
  if (mask_kind == SDPA_MASK_ADDITIVE && (rc = check_view("mask", x.ms, B, Hq, Lq, Lk)) != SDPA_OK) return rc;
  if (x.ks.l * es >= (int64_t(1) << 26) || x.vs.l * es >= (int64_t(1) << 26))
    return fail(SDPA_ERR_UNSUPPORTED, "k and v row strides must be below 2^26 bytes");
  if (p.route == SDPA_ROUTE_EMPTY) return SDPA_OK;
  if (!out) return fail(SDPA_ERR_INVALID, "out must not be NULL");
  if (!x.q) return fail(SDPA_ERR_INVALID, "q must not be NULL");
  if ((uintptr_t)out & 15) return fail(SDPA_ERR_INVALID, "q and out must be 16-byte aligned");
  if ((rc = check_rows_aligned("q", x.q, x.qs, es)) != SDPA_OK) return rc;
  if (mask_kind == SDPA_MASK_ADDITIVE && ((uintptr_t)x.mask % es))
    return fail(SDPA_ERR_INVALID, "an additive mask must be aligned to its element size");
  hipStream_t stream = (hipStream_t)stream_v;
  hipError_t e;
  if (p.route == SDPA_ROUTE_ZERO_FILL) {
    e = launch_zero_fill(out, B * Hq * Lq * Dv * es, stream);
    if (e != hipSuccess) return fail(SDPA_ERR_HIP, "zero-fill launch failed: %s", hipGetErrorString(e));
    return SDPA_OK;
  }
  if (!x.k || !x.v) return fail(SDPA_ERR_INVALID, "k and v must not be NULL");
  if ((rc = check_rows_aligned("k", x.k, x.ks, es)) != SDPA_OK) return rc;
  if ((rc = check_rows_aligned("v", x.v, x.vs, es)) != SDPA_OK) return rc;

  FwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = x.q;
  a.k = x.k;
  a.v = x.v;
  a.out = out;
  a.mask = mask_kind == SDPA_MASK_BOOL ? (const uint8_t*)x.mask : nullptr;
  a.sinks = sinks;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Lq = (int)Lq;
  a.Lk = (int)Lk;
  a.group = (int)(Hq / Hkv);
  a.mask_kind = mask_kind;
  a.window = (int)window;
  const Strides* st[3] = {&x.qs, &x.ks, &x.vs};
  int64_t* dst[3] = {a.qs, a.ks, a.vs};
  for (int i = 0; i < 3; ++i) {
    dst[i][0] = st[i]->b;
    dst[i][1] = st[i]->h;
    dst[i][2] = st[i]->l;
  }
  if (mask_kind == SDPA_MASK_ADDITIVE) {
    a.amask = x.mask;
    a.ms[0] = x.ms.b;
    a.ms[1] = x.ms.h;
    a.ms[2] = x.ms.l;
  }
  // scores are used in base 2; a zero scale becomes the smallest normal float,
  // which leaves every finite score's weight at exactly exp2(0) = 1
  a.c = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
  a.qsign = scale < 0.0f ? (dtype == SDPA_F32 ? 0x80000000u : 0x80008000u) : 0u;

  bool ok = false;
  if (p.route == SDPA_ROUTE_DECODE) {
    a.rows = (int)(a.group * Lq);
    a.koff = (int)window_first_key(Lq, Lk, window);
    a.kps = (int)p.keys_per_split;
    a.nsplit = (int)p.splits;
    void* part = nullptr;
    if ((rc = call_scratch(scratch_source, stream, (size_t)p.scratch_bytes, &part)) != SDPA_OK) return rc;
    a.part = (float*)part;
    DecodeShape s{p.rows_per_wave, p.waves, p.block_n};
    e = launch_decode(dtype, (int)D, (int)Dv, s, a, stream, &ok);
  } else {
    a.head_blocks = (int)(B * Hq / p.heads_per_group);
    a.nqb = (int)(p.grid[0] / a.head_blocks);
    // the plan gives the packing kernel scratch for the mask bits; the key-split
    // kernel reads the bytes itself
    if (prefill_packs_mask(dtype, mask_kind) && p.scratch_bytes > 0) {
      void* bits = nullptr;
      if ((rc = call_scratch(scratch_source, stream, (size_t)p.scratch_bytes, &bits)) != SDPA_OK) return rc;
      e = launch_mask_bits((const uint8_t*)x.mask, (uint32_t*)bits, Lq, Lk, stream);
      if (e != hipSuccess) return fail(SDPA_ERR_HIP, "mask packing launch failed: %s", hipGetErrorString(e));
      a.mbits = (const uint32_t*)bits;
      a.mwords = (int)mask_words(Lk);
    }
    PrefillShape s{p.rows_per_wave, p.waves, p.heads_per_group, p.block_n,
                   (int)((p.waves / p.heads_per_group) * p.rows_per_wave), (int)p.splits};
    e = launch_prefill(dtype, (int)D, (int)Dv, s, a, stream, &ok);
  }
  if (!ok) return fail(SDPA_ERR_UNSUPPORTED, "no kernel built for dtype %d, D=%lld, Dv=%lld", dtype, (long long)D,
                       (long long)Dv);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

// The views of a contiguous call.
Views contiguous_views(const void* q, const void* k, const void* v, const void* mask, int64_t Hq, int64_t Hkv,
                       int64_t Lq, int64_t Lk, int64_t D, int64_t Dv) {
  Views x;
  x.q = q;
  x.k = k;
  x.v = v;
  x.qs = contiguous(Hq, Lq, D);
  x.ks = contiguous(Hkv, Lk, D);
  x.vs = contiguous(Hkv, Lk, Dv);
  x.mask = mask;
  x.ms = Strides{0, 0, Lk};
  return x;
}

}  // namespace

extern "C" {

int sdpa_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t Hq, int64_t Hkv,
                 int64_t Lq, int64_t Lk, int64_t D, int64_t Dv, float scale, int mask_kind, const uint8_t* mask,
                 const void* sinks, int dtype, void* stream) {
  g_err.clear();
  if (mask_kind == SDPA_MASK_ADDITIVE)
    return fail(SDPA_ERR_INVALID, "an additive mask needs its strides: call sdpa_forward_strided");
  return forward_impl(contiguous_views(q, k, v, mask, Hq, Hkv, Lq, Lk, D, Dv), out, B, Hq, Hkv, Lq, Lk, D, Dv, scale,
                      mask_kind, sinks, dtype, 0, stream);
}

int sdpa_forward_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t Lq, int64_t Lk, int64_t D, int64_t Dv, float scale, int mask_kind,
                         const uint8_t* mask, const void* sinks, int dtype, void* stream) {
  g_err.clear();
  if (mask_kind == SDPA_MASK_ADDITIVE)
    return fail(SDPA_ERR_INVALID, "an additive mask needs its strides: call sdpa_forward_strided");
  return forward_impl(contiguous_views(q, k, v, mask, Hq, Hkv, Lq, Lk, D, Dv), out, B, Hq, Hkv, Lq, Lk, D, Dv, scale,
                      mask_kind, sinks, dtype, 0, stream, kScratchFixed);
}

int64_t sdpa_noalloc_scratch_bytes(void) { return (int64_t)kNoAllocScratchBytes; }

int sdpa_forward_windowed(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t Dv, float scale, int64_t window,
                          const void* sinks, int dtype, void* stream) {
  g_err.clear();
  int64_t w = 0;
  const int rc = effective_window(window, Lk, &w);
  if (rc != SDPA_OK) return rc;
  return forward_impl(contiguous_views(q, k, v, nullptr, Hq, Hkv, Lq, Lk, D, Dv), out, B, Hq, Hkv, Lq, Lk, D, Dv,
                      scale, SDPA_MASK_CAUSAL, sinks, dtype, w, stream);
}

int sdpa_plan_windowed(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t Dv,
                       int64_t window, int has_sinks, int dtype, sdpa_plan_t* plan) {
  g_err.clear();
  if (!plan) return fail(SDPA_ERR_INVALID, "plan must not be NULL");
  int64_t w = 0;
  int rc = effective_window(window, Lk, &w);
  if (rc != SDPA_OK) return rc;
  sdpa_plan_t p;
  rc = validate_and_plan(B, Hq, Hkv, Lq, Lk, D, Dv, SDPA_MASK_CAUSAL, false, has_sinks != 0, dtype, w, &p);
  if (rc == SDPA_OK) *plan = p;
  return rc;
}

}  // extern "C"

namespace {

// Validation and plan of a paged call (decode route only); fills `plan`.
int validate_and_plan_paged(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t D, int64_t Dv,
                            int64_t blocks, int64_t bs, int64_t max_blocks, int mask_kind, int64_t window,
                            int dtype, sdpa_plan_t* plan) {
  if (mask_kind != SDPA_MASK_NONE && mask_kind != SDPA_MASK_CAUSAL)
    return fail(SDPA_ERR_INVALID, "paged attention takes mask_kind 0 (none) or 1 (causal) (got %d)", mask_kind);
  if (window < 0) return fail(SDPA_ERR_INVALID, "window must be 0 (none) or >= 1 (got %lld)", (long long)window);
  if (window > 0 && mask_kind != SDPA_MASK_CAUSAL)
    return fail(SDPA_ERR_INVALID, "a window needs mask_kind SDPA_MASK_CAUSAL");
  if (blocks < 1) return fail(SDPA_ERR_INVALID, "blocks must be >= 1 (got %lld)", (long long)blocks);
  if (bs < 1) return fail(SDPA_ERR_INVALID, "bs must be >= 1 (got %lld)", (long long)bs);
  if (max_blocks < 1) return fail(SDPA_ERR_INVALID, "max_blocks must be >= 1 (got %lld)", (long long)max_blocks);
  int64_t cap;
  if (__builtin_mul_overflow(max_blocks, bs, &cap) || cap > kMaxLen)
    return fail(SDPA_ERR_UNSUPPORTED, "capacity max_blocks * bs exceeds %lld", (long long)kMaxLen);
  if (blocks > INT_MAX) return fail(SDPA_ERR_UNSUPPORTED, "blocks (%lld) exceeds INT_MAX", (long long)blocks);
  if (window > kMaxLen)
    return fail(SDPA_ERR_UNSUPPORTED, "window (%lld) exceeds %lld", (long long)window, (long long)kMaxLen);
  // the q / out / dtype / head checks of the contiguous call, with Lk = the capacity
  sdpa_plan_t p;
  int rc = validate_and_plan(B, Hq, Hkv, Lq, cap, D, Dv, mask_kind, false, false, dtype, 0, &p);
  if (rc != SDPA_OK) return rc;
  int64_t n;
  const int64_t es = elem_size(dtype);
  if (!mul4(blocks, Hkv, bs, D > Dv ? D : Dv, &n) || __builtin_mul_overflow(n, es, &n))
    return fail(SDPA_ERR_INVALID, "shape overflow: cache bytes do not fit in 64 bits");
  if (!mul3(B, max_blocks, 4, &n)) return fail(SDPA_ERR_INVALID, "shape overflow: table bytes do not fit in 64 bits");
  if (p.route == SDPA_ROUTE_EMPTY || dtype == SDPA_F32) {
    // f32: the f32 prefill kernel over the capacity's key range, any Lq
    *plan = p;
    return SDPA_OK;
  }
  const int64_t group = Hq / Hkv;
  if (Lq > 8 || group * Lq > 32)
    return fail(SDPA_ERR_UNSUPPORTED, "paged attention runs the decode kernels: Lq (%lld) <= 8 and "
                "(Hq/Hkv)*Lq (%lld) <= 32 needed", (long long)Lq, (long long)(group * Lq));
  // key splits from the capacity (lengths stay on the device), or from the
  // keys a window lets the rows read
  int64_t nkeys = cap;
  if (window > 0 && window + Lq - 1 < nkeys) nkeys = window + Lq - 1;
  const int64_t kps = keys_per_split(nkeys);
  const int64_t nsplit = (nkeys + kps - 1) / kps;
  const int64_t rows = group * Lq;
  p.route = SDPA_ROUTE_DECODE;
  p.kernels = 2;
  p.rows_per_wave = decode_mf((int)D, (int)rows);
  p.waves = kDecodeWaves;
  p.block_n = kDecodeBN;
  p.heads_per_group = (int32_t)group;
  p.keys_per_split = kps;
  p.splits = nsplit;
  p.grid[0] = nsplit;
  p.grid[1] = Hkv;
  p.grid[2] = B;
  if (Hkv > kMaxGridYZ || B > kMaxGridYZ)
    return fail(SDPA_ERR_UNSUPPORTED, "decode grid: Hkv (%lld) and B (%lld) must be <= 65535", (long long)Hkv,
                (long long)B);
  int64_t sb;
  if (!mul4(B * Hkv, nsplit, rows, (Dv + 4) * 4, &sb)) return fail(SDPA_ERR_INVALID, "decode scratch size overflows");
  p.scratch_bytes = sb;
  *plan = p;
  return SDPA_OK;
}

}  // namespace

extern "C" {

int sdpa_plan_paged(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t D, int64_t Dv, int64_t blocks,
                    int64_t bs, int64_t max_blocks, int mask_kind, int64_t window, int has_sinks, int dtype,
                    sdpa_plan_t* plan) {
  g_err.clear();
  (void)has_sinks;
  if (!plan) return fail(SDPA_ERR_INVALID, "plan must not be NULL");
  sdpa_plan_t p;
  const int rc = validate_and_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks, mask_kind, window, dtype, &p);
  if (rc == SDPA_OK) *plan = p;
  return rc;
}

int sdpa_paged_forward(const void* q, const void* kcache, const void* vcache, void* out, const int32_t* table,
                       const int32_t* lengths, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t D,
                       int64_t Dv, int64_t blocks, int64_t bs, int64_t max_blocks, float scale, int mask_kind,
                       int64_t window, const void* sinks, int dtype, void* stream_v) {
  g_err.clear();
  sdpa_plan_t p;
  int rc = validate_and_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks, mask_kind, window, dtype, &p);
  if (rc != SDPA_OK) return rc;
  if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  if (p.route == SDPA_ROUTE_EMPTY) return SDPA_OK;
  if (!out || !q) return fail(SDPA_ERR_INVALID, "q and out must not be NULL");
  if (!kcache || !vcache) return fail(SDPA_ERR_INVALID, "kcache and vcache must not be NULL");
  if (!table || !lengths) return fail(SDPA_ERR_INVALID, "table and lengths must not be NULL");
  if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)kcache | (uintptr_t)vcache) & 15)
    return fail(SDPA_ERR_INVALID, "q, kcache, vcache and out must be 16-byte aligned");
  if (((uintptr_t)table | (uintptr_t)lengths) & 3)
    return fail(SDPA_ERR_INVALID, "table and lengths must be 4-byte aligned");
  hipStream_t stream = (hipStream_t)stream_v;
  FwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = kcache;
  a.v = vcache;
  a.out = out;
  a.sinks = sinks;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Lq = (int)Lq;
  a.Lk = (int)(max_blocks * bs);
  a.group = (int)(Hq / Hkv);
  a.mask_kind = mask_kind;
  a.window = (int)window;
  a.table = table;
  a.lengths = lengths;
  a.blocks = (int)blocks;
  a.bs = (int)bs;
  a.max_blocks = (int)max_blocks;
  a.c = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
  a.qsign = scale < 0.0f ? (dtype == SDPA_F32 ? 0x80000000u : 0x80008000u) : 0u;
  a.qs[0] = Hq * Lq * D;
  a.qs[1] = Lq * D;
  a.qs[2] = D;
  bool ok = false;
  hipError_t e;
  if (p.route == SDPA_ROUTE_PREFILL) {
    a.head_blocks = (int)(B * Hq / p.heads_per_group);
    a.nqb = (int)(p.grid[0] / a.head_blocks);
    PrefillShape s{p.rows_per_wave, p.waves, p.heads_per_group, p.block_n,
                   (int)((p.waves / p.heads_per_group) * p.rows_per_wave), (int)p.splits};
    e = launch_prefill_f32_paged((int)D, (int)Dv, s, a, stream, &ok);
    if (!ok) return fail(SDPA_ERR_UNSUPPORTED, "no kernel built for dtype %d, D=%lld, Dv=%lld", dtype, (long long)D,
                         (long long)Dv);
    if (e != hipSuccess) return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SDPA_OK;
  }
  a.rows = (int)(a.group * Lq);
  a.kps = (int)p.keys_per_split;
  a.nsplit = (int)p.splits;
  void* part = nullptr;
  if ((rc = get_scratch(stream, (size_t)p.scratch_bytes, &part)) != SDPA_OK) return rc;
  a.part = (float*)part;
  DecodeShape s{p.rows_per_wave, p.waves, p.block_n};
  e = launch_decode_paged(dtype, (int)D, (int)Dv, s, a, stream, &ok);
  if (!ok) return fail(SDPA_ERR_UNSUPPORTED, "no kernel built for dtype %d, D=%lld, Dv=%lld", dtype, (long long)D,
                       (long long)Dv);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

int sdpa_paged_write(void* cache, const void* rows, const int32_t* slots, int64_t n, int64_t blocks, int64_t Hkv,
                     int64_t bs, int64_t E, int dtype, void* stream) {
  g_err.clear();
  if (dtype != SDPA_F32 && dtype != SDPA_F16 && dtype != SDPA_BF16)
    return fail(SDPA_ERR_INVALID, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16 (got %d)", dtype);
  if (n < 0) return fail(SDPA_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
  if (blocks < 0) return fail(SDPA_ERR_INVALID, "blocks must be >= 0 (got %lld)", (long long)blocks);
  if (Hkv < 0) return fail(SDPA_ERR_INVALID, "Hkv must be >= 0 (got %lld)", (long long)Hkv);
  if (bs < 1) return fail(SDPA_ERR_INVALID, "bs must be >= 1 (got %lld)", (long long)bs);
  if (E < 0) return fail(SDPA_ERR_INVALID, "E must be >= 0 (got %lld)", (long long)E);
  int64_t row_bytes, nb;
  if (__builtin_mul_overflow(E, (int64_t)elem_size(dtype), &row_bytes) || !mul4(blocks, Hkv, bs, row_bytes, &nb) ||
      !mul3(n, Hkv, row_bytes, &nb))
    return fail(SDPA_ERR_INVALID, "shape overflow: cache or row bytes do not fit in 64 bits");
  if (row_bytes % 16 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "a cache row (E * element size = %lld bytes) must be a multiple of 16 bytes",
                (long long)row_bytes);
  if (n == 0 || Hkv == 0 || E == 0) return SDPA_OK;
  if (!cache || !rows || !slots) return fail(SDPA_ERR_INVALID, "cache, rows and slots must not be NULL");
  if ((((uintptr_t)cache | (uintptr_t)rows) & 15) || ((uintptr_t)slots & 3))
    return fail(SDPA_ERR_INVALID, "cache and rows must be 16-byte aligned, slots 4-byte aligned");
  const hipError_t e = launch_paged_write(cache, rows, slots, n, blocks, Hkv, bs, row_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "paged write launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

int sdpa_forward_strided(const sdpa_view_t* q, const sdpa_view_t* k, const sdpa_view_t* v, void* out, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t Dv, float scale,
                         int mask_kind, const sdpa_view_t* mask, const void* sinks, int64_t window, int dtype,
                         void* stream) {
  g_err.clear();
  if (!q || !k || !v) return fail(SDPA_ERR_INVALID, "the q, k and v views must not be NULL");
  int64_t w = 0;
  if (window != 0) {
    if (mask_kind != SDPA_MASK_CAUSAL)
      return fail(SDPA_ERR_INVALID, "a window needs mask_kind SDPA_MASK_CAUSAL (got %d)", mask_kind);
    const int rc = effective_window(window, Lk, &w);
    if (rc != SDPA_OK) return rc;
  }
  Views x;
  x.q = q->data;
  x.k = k->data;
  x.v = v->data;
  x.qs = Strides{q->stride_b, q->stride_h, q->stride_l};
  x.ks = Strides{k->stride_b, k->stride_h, k->stride_l};
  x.vs = Strides{v->stride_b, v->stride_h, v->stride_l};
  x.mask = nullptr;
  x.ms = Strides{0, 0, 0};
  if (mask_kind == SDPA_MASK_BOOL || mask_kind == SDPA_MASK_ADDITIVE) {
    if (!mask || !mask->data) return fail(SDPA_ERR_INVALID, "mask_kind %d needs a mask view", mask_kind);
    x.mask = mask->data;
    x.ms = Strides{mask->stride_b, mask->stride_h, mask->stride_l};
    if (mask_kind == SDPA_MASK_BOOL && (x.ms.b != 0 || x.ms.h != 0 || x.ms.l != Lk))
      return fail(SDPA_ERR_UNSUPPORTED, "a boolean mask is one contiguous [Lq, Lk] matrix (strides 0, 0, Lk)");
  }
  return forward_impl(x, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, sinks, dtype, w, stream);
}

int sdpa_release_workspace(void) {
  g_err.clear();
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  int rc = SDPA_OK;
  auto release = [&](int dev, void* ptr) {
    hipError_t e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipFree(ptr);
    if (e != hipSuccess && rc == SDPA_OK) rc = fail(SDPA_ERR_HIP, "releasing scratch: %s", hipGetErrorString(e));
  };
  for (auto& kv : g_scratch)
    if (kv.second.ptr) release(kv.first.first, kv.second.ptr);
  for (auto& r : g_retired) release(r.first, r.second);
  g_scratch.clear();
  g_retired.clear();
  (void)hipSetDevice(cur);
  return rc;
}

}  // extern "C"
