// Attention backward, bf16, head dimensions 32 and 64, with and without
// dropout.  The kernel templates are in fa_bwd_bf16.h; head dimension 128 is
// instantiated in fa_bwd_bf16_d128.hip, which is compiled with other flags.
#include "fa_bwd_bf16.h"

namespace fa {

hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, int phases, int d,
                           hipStream_t stream) {
  if (d == 32)
    return a.drop.t < 256 ? dispatch<32, true>(a, causal, phases, stream)
                          : dispatch<32, false>(a, causal, phases, stream);
  if (d == 128) return launch_bwd_bf16_d128(a, causal, phases, stream);
  return a.drop.t < 256 ? dispatch<64, true>(a, causal, phases, stream)
                        : dispatch<64, false>(a, causal, phases, stream);
}

}  // namespace fa
