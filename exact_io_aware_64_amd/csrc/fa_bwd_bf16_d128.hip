// Attention backward, bf16, head dimension 128, with and without dropout.  The kernel
// templates are in fa_bwd_bf16.h.  This file is compiled without the flag that
// keeps MFMA accumulators in the architectural VGPRs: at one wave per SIMD the
// dK/dV role's accumulators (64 KB of dK^T and dV^T per wave) then live in the
// accumulation registers, beside the 256 VGPRs, and no item has to recompute S
// and dP to split the output columns.
#include "fa_bwd_bf16.h"

namespace fa {

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, bool causal, int phases,
                                hipStream_t stream) {
  return a.drop.t < 256 ? dispatch<128, true>(a, causal, phases, stream)
                        : dispatch<128, false>(a, causal, phases, stream);
}

}  // namespace fa
