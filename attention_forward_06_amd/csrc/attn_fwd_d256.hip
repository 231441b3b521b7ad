// Attention forward for AMD Instinct MI355X (gfx950): the head-dim-256 instances (none and
// causal; fp16 or bf16 Q/K/O with 16-bit or OCP e5m2 V -- "Fused Attention", _attn_fwd_inner,
// HEAD_DIM 256 and the fp8 branch).
//
// This unit is built with the MFMA accumulators held in VGPRs (-mllvm -amdgpu-mfma-vgpr-form).
// At head dim 256 a wave's state exceeds 256 registers (one wave per SIMD), so the compiler
// otherwise keeps O in AGPRs, and every VALU touch of O -- the fp8 recurrence rescales it at
// every increase of a row's running maximum -- round-trips it through VGPRs (measured on one
// GPU: ~430 AGPR copy instructions per iteration; 13% slower on causal L = 32768 with e5m2 V).
// Q's fragments, which only MFMAs read, go to AGPRs instead.  The other head dims run two
// waves per SIMD within 256 VGPRs and stay in attn_fwd.hip.
#include "attn_kernel.h"

namespace {

template <int DT>
hipError_t dispatch_d256(int mode, const Params& p, hipStream_t s) {
  if (mode == kMaskCausal) return launch<256, DT, kMaskCausal, 4, 64>(p, s);
  return launch<256, DT, kMaskNone, 4, 64>(p, s);
}

}  // namespace

namespace attn {

int launch_d256(const Problem& pr, const LaunchArgs& a, void* stream) {
  const Params p = make_params(a);
  hipStream_t s = (hipStream_t)stream;
  switch (pr.dtype) {
    case kF16: return (int)dispatch_d256<kF16>(pr.mode, p, s);
    case kBF16: return (int)dispatch_d256<kBF16>(pr.mode, p, s);
    case kF16V8: return (int)dispatch_d256<kF16V8>(pr.mode, p, s);
    default: return (int)dispatch_d256<kBF16V8>(pr.mode, p, s);
  }
}

}  // namespace attn
