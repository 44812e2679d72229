// Prefill kernel instantiations for 16-bit inputs (bf16 and f16).
#include "prefill_fast.h"
#include "prefill_impl.h"
#include "prefill_ksplit.h"

namespace sdpa {

template <class E, int D, int DV>
static hipError_t launch_one(const PrefillShape& s, const FwdArgs& a, hipStream_t stream) {
  constexpr int elem = std::is_same<E, ElemBF16>::value ? kBF16 : kF16;
  dim3 grid(a.head_blocks * a.nqb, 1, 1);
  if constexpr (prefill_can_ksplit(elem, D, DV)) {
    using C = KsplitCfg<D, DV>;
    static_assert(C::MF == kKsplitRows && C::SUB == kKsplitBN && C::KL == kKsplitLanes && C::NWH == kPrefillWaves,
                  "planner geometry must match the kernel");
    // the plan chose the key-split kernel (every call with heads of 192 columns or
    // more, 128-wide calls with an additive mask, narrower heads on small grids)
    if (s.ksplit > 1) {
      if (s.ksplit != C::KL || s.mf != C::MF || s.block_n != C::SUB || s.waves != C::NW)
        return hipErrorInvalidConfiguration;
      if (a.mask_kind == kMaskBool)
        hipLaunchKernelGGL((prefill_ksplit_kernel<E, D, DV, kKsBool>), grid, dim3(C::NW * 64), 0, stream, a);
      else if (a.mask_kind == kMaskAdditive)
        hipLaunchKernelGGL((prefill_ksplit_kernel<E, D, DV, kKsAdd>), grid, dim3(C::NW * 64), 0, stream, a);
      else
        hipLaunchKernelGGL((prefill_ksplit_kernel<E, D, DV, kKsPlain>), grid, dim3(C::NW * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  if (s.ksplit > 1) return hipErrorInvalidConfiguration;
  if constexpr (prefill_can_ksplit(elem, D, DV) && prefill_ksplit_always(D, DV, kMaskNone)) {
    return hipErrorInvalidConfiguration;   // these 16-bit heads run the key-split kernel only
  } else {
    constexpr int MF = prefill_generic_mf(elem, D, DV);
    constexpr int BN = prefill_generic_bn(elem, D, DV);
    if (a.mask_kind == kMaskAdditive) {
      hipLaunchKernelGGL((prefill_kernel<E, MF, D, DV, BN, kPrefillWaves, true>), grid, dim3(kPrefillWaves * 64), 0,
                         stream, a);
      return hipGetLastError();
    }
    if constexpr (prefill_can_fast(elem, D, DV, kMaskNone)) {
      // the pipelined kernel (32-row tiles)
      using C = FastCfg<D, DV>;
      static_assert(C::MF == kFastRows && C::ROWS == kFastRows && C::BN == kFastBN && C::NW == kPrefillWaves,
                    "planner geometry must match the kernel");
      if (s.mf != C::MF || s.block_n != C::BN) return hipErrorInvalidConfiguration;
      if (a.mask_kind == kMaskBool)
        hipLaunchKernelGGL((prefill_fast_kernel<E, D, DV, true>), grid, dim3(C::NW * 64), 0, stream, a);
      else
        hipLaunchKernelGGL((prefill_fast_kernel<E, D, DV, false>), grid, dim3(C::NW * 64), 0, stream, a);
      return hipGetLastError();
    } else {
      hipLaunchKernelGGL((prefill_kernel<E, MF, D, DV, BN, kPrefillWaves, false>), grid, dim3(kPrefillWaves * 64), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
}

hipError_t launch_prefill_16(int elem, int D, int Dv, const PrefillShape& s, const FwdArgs& a,
                             hipStream_t stream, bool* ok) {
  *ok = true;
#define SDPA_PAIR(d, dv)                                                   \
  if (D == d && Dv == dv)                                                  \
    return elem == kBF16 ? launch_one<ElemBF16, d, dv>(s, a, stream)      \
                         : launch_one<ElemF16, d, dv>(s, a, stream);
  SDPA_HEAD_PAIRS(SDPA_PAIR)
#undef SDPA_PAIR
  *ok = false;
  return hipSuccess;
}

}  // namespace sdpa
