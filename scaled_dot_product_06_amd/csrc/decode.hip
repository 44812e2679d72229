// Decode (split-key first pass + log-sum-exp reduce) instantiations, 16-bit inputs.
#include "decode_impl.h"

namespace sdpa {

template <class E, int D, int DV>
static hipError_t launch_one(const DecodeShape& s, const FwdArgs& a, hipStream_t stream) {
  dim3 grid1(a.nsplit, a.Hkv, a.B);
  if constexpr (D % 32 == 0) {
    if (s.mf == 16) {
      hipLaunchKernelGGL((decode_split_kernel<E, 16, D, DV, kDecodeWaves>), grid1, dim3(kDecodeWaves * 64), 0,
                         stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 grid2(a.rows, a.Hkv, a.B * (DV / reduce_cols(DV)));
      hipLaunchKernelGGL((decode_reduce_kernel<E, DV>), grid2, dim3(256), 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_split_kernel<E, 32, D, DV, kDecodeWaves>), grid1, dim3(kDecodeWaves * 64), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.rows, a.Hkv, a.B * (DV / reduce_cols(DV)));
  hipLaunchKernelGGL((decode_reduce_kernel<E, DV>), grid2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(int elem, int D, int Dv, const DecodeShape& s, const FwdArgs& a, hipStream_t stream,
                         bool* ok) {
  *ok = true;
  if (elem != kBF16 && elem != kF16) {
    *ok = false;
    return hipSuccess;
  }
#define SDPA_PAIR(d, dv)                                                 \
  if (D == d && Dv == dv)                                                \
    return elem == kBF16 ? launch_one<ElemBF16, d, dv>(s, a, stream)    \
                         : launch_one<ElemF16, d, dv>(s, a, stream);
  SDPA_HEAD_PAIRS(SDPA_PAIR)
#undef SDPA_PAIR
  *ok = false;
  return hipSuccess;
}

}  // namespace sdpa
