// Attention forward for AMD Instinct MI355X (gfx950): the instances of head dims 16-128 (none
// and causal) and of block_diag, and the host-side launch of a validated call.  Head dims 16-64
// (none and causal) run attn_fwd_rows64_kernel (attn_kernel_rows64.h), head dim 128 and
// block_diag attn_fwd_kernel (attn_kernel.h); the head-dim-256 instances are in
// attn_fwd_d256.hip.
#include "attn_kernel.h"
#include "attn_kernel_rows64.h"

namespace {

template <int D, int DT>
hipError_t dispatch_dense(int mode, const Params& p, hipStream_t s) {
  // 4 waves (128 query rows) per workgroup and 64-key tiles for every head dim: two waves per
  // SIMD fit the register budget, two workgroups per CU interleave their MFMA and VALU phases.
  if (mode == kMaskCausal) return launch<D, DT, kMaskCausal, 4, 64>(p, s);
  return launch<D, DT, kMaskNone, 4, 64>(p, s);
}

template <int D, int DT>
hipError_t dispatch_block(int64_t bs, const Params& p, hipStream_t s) {
  // Every block size runs 128 query rows (4 waves) per workgroup: 128 / bs diagonal blocks
  // behind one 128-row K/V transfer (larger transfers keep more bytes in flight); each wave
  // works on the bs keys of its own block.
  if (bs == 32) return launch<D, DT, kMaskBlock, 4, 128, 32>(p, s);
  if (bs == 64) return launch<D, DT, kMaskBlock, 4, 128, 64>(p, s);
  return launch<D, DT, kMaskBlock, 4, 128, 128>(p, s);
}

hipError_t dispatch(const attn::Problem& pr, const Params& p, hipStream_t s) {
  if (pr.mode == kMaskBlock) {
    if (pr.D == 64) return pr.dtype == kF16 ? dispatch_block<64, kF16>(pr.block_size, p, s)
                                            : dispatch_block<64, kBF16>(pr.block_size, p, s);
    return pr.dtype == kF16 ? dispatch_block<128, kF16>(pr.block_size, p, s)
                            : dispatch_block<128, kBF16>(pr.block_size, p, s);
  }
  // head dims 16-64: 64 query rows per wave (attn_kernel_rows64.h)
  const bool causal = pr.mode == kMaskCausal;
  const bool f16 = pr.dtype == kF16;
  switch (pr.D) {
    case 16:
      if (causal) return f16 ? launch_rows64<16, kF16, kMaskCausal>(p, s) : launch_rows64<16, kBF16, kMaskCausal>(p, s);
      return f16 ? launch_rows64<16, kF16, kMaskNone>(p, s) : launch_rows64<16, kBF16, kMaskNone>(p, s);
    case 32:
      if (causal) return f16 ? launch_rows64<32, kF16, kMaskCausal>(p, s) : launch_rows64<32, kBF16, kMaskCausal>(p, s);
      return f16 ? launch_rows64<32, kF16, kMaskNone>(p, s) : launch_rows64<32, kBF16, kMaskNone>(p, s);
    case 64:
      if (causal) return f16 ? launch_rows64<64, kF16, kMaskCausal>(p, s) : launch_rows64<64, kBF16, kMaskCausal>(p, s);
      return f16 ? launch_rows64<64, kF16, kMaskNone>(p, s) : launch_rows64<64, kBF16, kMaskNone>(p, s);
    case 128:
      return pr.dtype == kF16 ? dispatch_dense<128, kF16>(pr.mode, p, s)
                              : dispatch_dense<128, kBF16>(pr.mode, p, s);
    default:
      return hipErrorInvalidValue;   // head dim 256: launch_d256
  }
}

}  // namespace

namespace attn {

int launch(const Problem& pr, const LaunchArgs& a, void* stream) {
  // head dim 256 (every dtype, none and causal): instances in attn_fwd_d256.hip
  if (pr.mode != kMaskBlock && pr.D == 256) return launch_d256(pr, a, stream);
  return (int)dispatch(pr, make_params(a), (hipStream_t)stream);
}

}  // namespace attn
