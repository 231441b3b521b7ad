// The C ABI of the attention forward (include/attn_fwd.h): argument checks and the conversion
// of a call into launch arguments.  Plain C++ with no HIP dependency: the kernels (attn_kernel.h)
// and their launch (attn_fwd.hip, attn_fwd_d256.hip) sit behind attn::launch, so this file also
// builds on its own with the host sanitizers.
#include <climits>
#include <cstdint>

#include "../../include/attn_fwd.h"
#include "attn_host.h"

namespace {

using attn::Layout;
using attn::LaunchArgs;
using attn::Problem;

constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskBlock = 2;
constexpr int kF16 = 0, kBF16 = 1, kBF16V8 = 2, kF16V8 = 3;
constexpr float kLog2e = 1.44269504088896340736f;
// Every tensor row, and every base the kernels address, sits on a 16-byte boundary: Q and O are
// moved 8 or 16 bytes per lane and K/V rows by 16-byte LDS-DMA chunks.
constexpr int64_t kAlign = 16;

bool supported(const Problem& pr) {
  const bool dense = pr.mode == kMaskNone || pr.mode == kMaskCausal;
  if (dense) {
    if (pr.D == 16 || pr.D == 32 || pr.D == 64 || pr.D == 128) return pr.dtype == kF16 || pr.dtype == kBF16;
    return pr.D == 256;
  }
  if (pr.D != 64 && pr.D != 128) return false;
  if (pr.dtype != kF16 && pr.dtype != kBF16) return false;
  return pr.block_size == 32 || pr.block_size == 64 || pr.block_size == 128;
}

attn_status_t validate(const Problem& pr) {
  if (pr.mode < kMaskNone || pr.mode > kMaskBlock || pr.dtype < kF16 || pr.dtype > kF16V8)
    return ATTN_ERR_ARG;
  // finite and positive, checked on the bits (independent of floating-point flags)
  const uint32_t sbits = __builtin_bit_cast(uint32_t, pr.sm_scale);
  const bool not_finite = ((sbits >> 23) & 0xffu) == 0xffu;
  if (not_finite || (sbits >> 31) != 0u || (sbits & 0x7fffffffu) == 0u) return ATTN_ERR_ARG;
  if (pr.batch < 0 || pr.heads < 0 || pr.L < 0 || pr.D <= 0) return ATTN_ERR_SHAPE;
  if (pr.mode == kMaskBlock) {
    if (pr.block_size <= 0) return ATTN_ERR_SHAPE;
    if (pr.L % pr.block_size != 0) return ATTN_ERR_SHAPE;
  }
  // Sizes: every count must fit the kernels' index types.
  const int64_t lim = (int64_t)1 << 31;
  if (pr.L >= lim || pr.batch >= lim || pr.heads >= lim || pr.D >= lim) return ATTN_ERR_SHAPE;
  const int64_t bh = pr.batch * pr.heads;                      // < 2^62: no overflow
  if (bh >= lim) return ATTN_ERR_SHAPE;
  if (pr.L * pr.D * 2 >= lim) return ATTN_ERR_SHAPE;           // one head must fit 2^31 bytes
  if (((pr.L + 31) / 32) * bh >= lim) return ATTN_ERR_SHAPE;   // workgroup count fits the grid
  if (!supported(pr)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// One tensor's element strides (batch, head, row; D contiguous): non-negative, rows at least D
// apart (so row L of a head starts past the head's last element, which the kernels rely on to
// read rows past L as zeros), every stride a whole number of 16-byte units, one head's rows
// within 2^31 bytes (32-bit buffer offsets), and every element offset within int64.  Called
// after validate(), so the sizes are bounded as checked there.
attn_status_t validate_layout(const Problem& pr, const int64_t* st, int64_t elem_bytes) {
  const int64_t sb = st[0], sh = st[1], sr = st[2];
  const int64_t lim = (int64_t)1 << 31;
  if (sb < 0 || sh < 0 || sr < pr.D || sr >= lim) return ATTN_ERR_SHAPE;
  // strides in bytes on 16-byte boundaries (sb, sh < 2^63 / 2: the products cannot overflow
  // once checked against INT64_MAX / elem_bytes)
  if (sb > INT64_MAX / elem_bytes || sh > INT64_MAX / elem_bytes) return ATTN_ERR_SHAPE;
  if ((sb * elem_bytes) % kAlign != 0 || (sh * elem_bytes) % kAlign != 0 ||
      (sr * elem_bytes) % kAlign != 0)
    return ATTN_ERR_SHAPE;
  if (pr.batch == 0 || pr.heads == 0 || pr.L == 0) return ATTN_OK;
  const __int128 extent = ((__int128)(pr.L - 1) * sr + pr.D) * elem_bytes;
  if (extent >= lim) return ATTN_ERR_SHAPE;
  const __int128 last = (__int128)(pr.batch - 1) * sb + (__int128)(pr.heads - 1) * sh + extent / elem_bytes;
  if (last * elem_bytes > (__int128)INT64_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

}  // namespace

extern "C" {

attn_status_t attn_fwd_check(int64_t batch, int64_t heads, int64_t L, int64_t D, float sm_scale,
                             attn_mask_t mask_mode, int64_t block_size, attn_dtype_t dtype) {
  const Problem pr{batch, heads, L, D, sm_scale, (int)mask_mode, block_size, (int)dtype};
  return validate(pr);
}

attn_status_t attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t batch, int64_t heads, int64_t L, int64_t D,
                               const int64_t* q_strides, const int64_t* k_strides,
                               const int64_t* v_strides, const int64_t* o_strides, float sm_scale,
                               attn_mask_t mask_mode, int64_t block_size, attn_dtype_t dtype,
                               void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (q_strides == nullptr || k_strides == nullptr || v_strides == nullptr || o_strides == nullptr)
    return ATTN_ERR_NULL;
  const Problem pr{batch, heads, L, D, sm_scale, (int)mask_mode, block_size, (int)dtype};
  attn_status_t st = validate(pr);
  if (st != ATTN_OK) return st;
  const int64_t vb = (dtype == ATTN_BF16_V_E5M2 || dtype == ATTN_F16_V_E5M2) ? 1 : 2;
  if ((st = validate_layout(pr, q_strides, 2)) != ATTN_OK) return st;
  if ((st = validate_layout(pr, k_strides, 2)) != ATTN_OK) return st;
  if ((st = validate_layout(pr, v_strides, vb)) != ATTN_OK) return st;
  if ((st = validate_layout(pr, o_strides, 2)) != ATTN_OK) return st;
  if (!aligned(q, kAlign) || !aligned(k, kAlign) || !aligned(v, kAlign) || !aligned(o, kAlign) ||
      !aligned(lse, 4))
    return ATTN_ERR_SHAPE;
  if (batch * heads * L == 0) return ATTN_OK;
  LaunchArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.lq = Layout{q_strides[0], q_strides[1], (int)q_strides[2]};
  a.lk = Layout{k_strides[0], k_strides[1], (int)k_strides[2]};
  a.lv = Layout{v_strides[0], v_strides[1], (int)v_strides[2]};
  a.lo = Layout{o_strides[0], o_strides[1], (int)o_strides[2]};
  a.heads = (int)heads;
  a.L = (int)L;
  a.bh = (int)(batch * heads);
  a.c = sm_scale * kLog2e;
  return attn::launch(pr, a, stream) == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t batch, int64_t heads, int64_t L, int64_t D, float sm_scale,
                           attn_mask_t mask_mode, int64_t block_size, attn_dtype_t dtype,
                           void* stream) {
  // contiguous [batch, heads, L, D]; the stride products are formed only for sizes that pass
  // validation (which bounds them far below int64)
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_NULL;
  const attn_status_t vs = validate(Problem{batch, heads, L, D, sm_scale, (int)mask_mode, block_size, (int)dtype});
  if (vs != ATTN_OK) return vs;
  const int64_t st[3] = {heads * L * D, L * D, D};
  return attn_fwd_strided(q, k, v, o, lse, batch, heads, L, D, st, st, st, st, sm_scale, mask_mode,
                          block_size, dtype, stream);
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t batch,
                       int64_t heads, int64_t L, int64_t D, float sm_scale, attn_mask_t mask_mode,
                       int64_t block_size, attn_dtype_t dtype, void* stream) {
  return attn_fwd_lse(q, k, v, o, nullptr, batch, heads, L, D, sm_scale, mask_mode, block_size,
                      dtype, stream);
}

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE:
      return "invalid shape or layout (negative size, overflow, block_size not dividing L, or a "
             "pointer or stride off a 16-byte boundary)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported (mask mode, head dim, dtype, block size) combination";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_ARG: return "invalid scalar argument (enum value or sm_scale)";
  }
  return "unknown status";
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
