// Attention forward for AMD Instinct MI355X (gfx950): the instances with OCP e5m2 V (head dim
// 256, bf16 or fp16 Q/K/O, none and causal; "Fused Attention", _attn_fwd_inner fp8 branch).
//
// This unit is built with the MFMA accumulators held in VGPRs (-mllvm -amdgpu-mfma-vgpr-form):
// the fp8 recurrence rescales O at every increase of a row's running maximum, and with O in
// AGPRs every rescale round-trips it through VGPRs (measured on one GPU: ~430 AGPR copy
// instructions per iteration, 13% slower on causal L = 32768).  The 16-bit-V instances stay in
// attn_fwd.hip, where the same flag measured 8% slower at head dim 256.
#include "attn_kernel.h"

namespace {

template <int DT>
hipError_t dispatch_v8(int mode, const Params& p, hipStream_t s) {
  if (mode == kMaskCausal) return launch<256, DT, kMaskCausal, 4, 64>(p, s);
  return launch<256, DT, kMaskNone, 4, 64>(p, s);
}

}  // namespace

namespace attn {

int launch_v8(const Problem& pr, const LaunchArgs& a, void* stream) {
  const Params p = make_params(a);
  if (pr.dtype == kF16V8) return (int)dispatch_v8<kF16V8>(pr.mode, p, (hipStream_t)stream);
  return (int)dispatch_v8<kBF16V8>(pr.mode, p, (hipStream_t)stream);
}

}  // namespace attn
