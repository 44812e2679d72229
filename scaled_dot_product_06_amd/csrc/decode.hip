// Decode (split-key first pass + log-sum-exp reduce) instantiations, 16-bit
// inputs, over contiguous K/V or paged caches; and the paged cache write.
#include "decode_impl.h"

namespace sdpa {

template <class E, int D, int DV, bool PAGED>
static hipError_t launch_one(const DecodeShape& s, const FwdArgs& a, hipStream_t stream) {
  dim3 grid1(a.nsplit, a.Hkv, a.B);
  bool done = false;
  if constexpr (D % 32 == 0) {
    if (s.mf == 16) {
      hipLaunchKernelGGL((decode_split_kernel<E, 16, D, DV, kDecodeWaves, PAGED>), grid1,
                         dim3(kDecodeWaves * 64), 0, stream, a);
      done = true;
    }
  }
  if (!done)
    hipLaunchKernelGGL((decode_split_kernel<E, 32, D, DV, kDecodeWaves, PAGED>), grid1, dim3(kDecodeWaves * 64),
                       0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.rows * (DV / reduce_cols(DV)), a.Hkv, a.B);
  hipLaunchKernelGGL((decode_reduce_kernel<E, DV>), grid2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool PAGED>
static hipError_t launch_any(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a, hipStream_t stream,
                             bool* ok) {
  *ok = true;
  if (elem != kBF16 && elem != kF16) {
    *ok = false;
    return hipSuccess;
  }
#define SDPA_PAIR(d, dv)                                                        \
  if (D == d && Dv == dv)                                                       \
    return elem == kBF16 ? launch_one<ElemBF16, d, dv, PAGED>(s, a, stream)    \
                         : launch_one<ElemF16, d, dv, PAGED>(s, a, stream);
  SDPA_HEAD_PAIRS(SDPA_PAIR)
#undef SDPA_PAIR
  *ok = false;
  return hipSuccess;
}

hipError_t launch_decode(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a, hipStream_t stream,
                         bool* ok) {
  return launch_any<false>(elem, D, Dv, s, a, stream, ok);
}

hipError_t launch_decode_paged(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a,
                               hipStream_t stream, bool* ok) {
  return launch_any<true>(elem, D, Dv, s, a, stream, ok);
}

// Paged cache write (nuvec-core "tests/fast.rs", paged_write_matches_the_
// fallback_and_writes_in_place, paged_write_skips_out_of_range_slots): row r
// of `rows` ([n, Hkv, row]) goes to slot slots[r] = block * bs + position of
// `cache` ([blocks, Hkv, bs, row]); a slot outside [0, blocks * bs) is skipped.
// One thread per 16-byte chunk of one (row, head), a grid-stride loop.
typedef uint32_t u32x4_w __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) paged_write_kernel(u32x4_w* cache, const u32x4_w* rows,
                                                         const int32_t* slots, int64_t n, int64_t blocks,
                                                         int64_t Hkv, int64_t bs, int64_t chunks) {
  const int64_t total = n * Hkv * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t c = i % chunks, rh = i / chunks, h = rh % Hkv, r = rh / Hkv;
    const int64_t slot = slots[r];
    if (slot < 0 || slot >= blocks * bs) continue;
    const int64_t dst = ((slot / bs) * Hkv + h) * bs + slot % bs;
    cache[dst * chunks + c] = rows[(r * Hkv + h) * chunks + c];
  }
}

hipError_t launch_paged_write(void* cache, const void* rows, const int32_t* slots, int64_t n, int64_t blocks,
                              int64_t Hkv, int64_t bs, int64_t row_bytes, hipStream_t stream) {
  const int64_t chunks = row_bytes / 16;
  int64_t grid = (n * Hkv * chunks + 255) / 256;
  if (grid > (1 << 16)) grid = 1 << 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(paged_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (u32x4_w*)cache,
                     (const u32x4_w*)rows, slots, n, blocks, Hkv, bs, chunks);
  return hipGetLastError();
}

}  // namespace sdpa
