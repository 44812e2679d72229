// Prefill kernel instantiations for float32 inputs (f32 MFMA).
#include "prefill_impl.h"

namespace sdpa {

template <int MF, int D, int DV>
static hipError_t launch_mf(const FwdArgs& a, hipStream_t stream) {
  constexpr int BN = prefill_generic_bn(kF32, D, DV);
  dim3 grid(a.head_blocks * a.nqb, 1, 1);
  if (a.mask_kind == kMaskAdditive)
    hipLaunchKernelGGL((prefill_f32_kernel<MF, D, DV, BN, kPrefillWaves, true>), grid, dim3(kPrefillWaves * 64), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<MF, D, DV, BN, kPrefillWaves, false>), grid, dim3(kPrefillWaves * 64),
                       0, stream, a);
  return hipGetLastError();
}

// The plan's kernel: the key-split one for small calls, else the generic
// walk with its tile height (16 rows for small paged or additive calls).
template <int D, int DV>
static hipError_t launch_one(const PrefillShape& s, const FwdArgs& a, hipStream_t stream) {
  constexpr int MF = prefill_generic_mf(kF32, D, DV);
  if constexpr (MF == 32) {
    if (s.ksplit > 1) {
      constexpr int BN = f32_split_bn(D, DV);
      if (s.ksplit != kPrefillWaves || s.block_n != BN || s.mf != 16 || a.mask_kind == kMaskAdditive)
        return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((prefill_f32_split_kernel<D, DV, BN, kPrefillWaves, false>), dim3(a.head_blocks * a.nqb),
                         dim3(kPrefillWaves * 64), 0, stream, a);
      return hipGetLastError();
    }
    if (s.mf == 16) return launch_mf<16, D, DV>(a, stream);
  }
  return launch_mf<MF, D, DV>(a, stream);
}

hipError_t launch_prefill_f32(int D, int Dv, const PrefillShape& s, const FwdArgs& a, hipStream_t stream,
                              bool* ok) {
  *ok = true;
#define SDPA_PAIR(d, dv) \
  if (D == d && Dv == dv) return launch_one<d, dv>(s, a, stream);
  SDPA_HEAD_PAIRS(SDPA_PAIR)
#undef SDPA_PAIR
  *ok = false;
  return hipSuccess;
}

template <int MF, int D, int DV>
static hipError_t launch_paged_mf(const FwdArgs& a, hipStream_t stream) {
  constexpr int BN = prefill_generic_bn(kF32, D, DV);
  dim3 grid(a.head_blocks * a.nqb, 1, 1);
  hipLaunchKernelGGL((prefill_f32_kernel<MF, D, DV, BN, kPrefillWaves, false, true>), grid,
                     dim3(kPrefillWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int DV>
static hipError_t launch_paged_one(const PrefillShape& s, const FwdArgs& a, hipStream_t stream) {
  constexpr int MF = prefill_generic_mf(kF32, D, DV);
  if constexpr (MF == 32) {
    if (s.ksplit > 1) {
      constexpr int BN = f32_split_bn(D, DV);
      if (s.ksplit != kPrefillWaves || s.block_n != BN || s.mf != 16) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((prefill_f32_split_kernel<D, DV, BN, kPrefillWaves, true>), dim3(a.head_blocks * a.nqb),
                         dim3(kPrefillWaves * 64), 0, stream, a);
      return hipGetLastError();
    }
    if (s.mf == 16) return launch_paged_mf<16, D, DV>(a, stream);
  }
  return launch_paged_mf<MF, D, DV>(a, stream);
}

hipError_t launch_prefill_f32_paged(int D, int Dv, const PrefillShape& s, const FwdArgs& a, hipStream_t stream,
                                    bool* ok) {
  *ok = true;
#define SDPA_PAIR(d, dv) \
  if (D == d && Dv == dv) return launch_paged_one<d, dv>(s, a, stream);
  SDPA_HEAD_PAIRS(SDPA_PAIR)
#undef SDPA_PAIR
  *ok = false;
  return hipSuccess;
}

}  // namespace sdpa
