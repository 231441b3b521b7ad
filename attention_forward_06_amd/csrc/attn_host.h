// Interface between the host-side argument checks (attn_api.cpp, plain C++ with no HIP
// dependency, so it can also be built with the host sanitizers) and the kernel launcher
// (attn_fwd.hip; head dim 256 in attn_fwd_d256.hip).  Not part of the public C ABI.
#pragma once

#include <cstdint>

namespace attn {

// Element strides of one [batch, heads, L, D] tensor; D is contiguous.
struct Layout {
  long long sb, sh;  // batch, head
  int sr;            // row (sequence position), >= D
};

// The call as the caller made it (sizes, scalars, enums as integers).
struct Problem {
  int64_t batch, heads, L, D;
  float sm_scale;
  int mode;  // attn_mask_t
  int64_t block_size;
  int dtype;  // attn_dtype_t
};

// A validated, non-empty problem in the form the kernels take.
struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // NULL: no log-normaliser output
  Layout lq, lk, lv, lo;
  int heads;
  int L;
  int bh;   // batch * heads
  float c;  // sm_scale * log2(e)
};

// Enqueue the forward for a problem that passed validation; returns 0 on success, else the
// HIP runtime's error code.  Implemented next to the kernels.
int launch(const Problem& pr, const LaunchArgs& a, void* stream);

// The same for head dim 256 in the streamed modes (its instances live in their own translation
// unit, built with MFMA accumulators in VGPRs).
int launch_d256(const Problem& pr, const LaunchArgs& a, void* stream);

}  // namespace attn
