// Host-only checks of the C ABI's argument handling (attn_api.cpp), built without HIP and meant
// to run under the host sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer).  The kernel
// launcher is replaced by a stub that records what it was given, so every entry point can be
// called with fake device pointers: rejected calls must never reach the launcher, accepted ones
// must reach it once with the sizes, strides and scale the caller passed.  Any signed overflow,
// shift or out-of-bounds access in the checks themselves is reported by the sanitizers.
//
// Build: g++ -std=c++17 -fsanitize=address,undefined host_checks.cpp attn_api.cpp
// Prints one summary line; exits non-zero on the first failed check.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "../../include/attn_fwd.h"
#include "attn_host.h"

namespace {

int g_calls = 0;
attn::Problem g_pr{};
attn::LaunchArgs g_args{};
int g_launch_result = 0;
long g_checks = 0;

void expect(bool ok, const char* what, long line) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "host check failed at line %ld: %s\n", line, what);
    std::exit(1);
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

constexpr int64_t I64MAX = std::numeric_limits<int64_t>::max();
constexpr int64_t I64MIN = std::numeric_limits<int64_t>::min();

attn_status_t strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t H, int64_t L, int64_t D, const int64_t* qs, const int64_t* ks,
                      const int64_t* vs, const int64_t* os, float scale, int mode, int64_t bs, int dt) {
  return attn_fwd_strided(q, k, v, o, lse, B, H, L, D, qs, ks, vs, os, scale, (attn_mask_t)mode, bs,
                          (attn_dtype_t)dt, nullptr);
}

// Deterministic 64-bit generator (splitmix64) for the randomised part.
uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
// A size drawn from small values, powers of two and the int64 extremes.
int64_t draw_size() {
  switch (next_u64() % 12) {
    case 0: return (int64_t)(next_u64() % 5);
    case 1: return (int64_t)(next_u64() % 600);
    case 2: return (int64_t)1 << (next_u64() % 63);
    case 3: return ((int64_t)1 << (next_u64() % 63)) - 1;
    case 4: return -(int64_t)(next_u64() % 1000);
    case 5: return (next_u64() & 1) ? I64MAX : I64MIN;
    case 6: return 16 * (int64_t)(next_u64() % 4096);
    case 7: return (int64_t)(next_u64() >> 1);
    default: return 1 + (int64_t)(next_u64() % 300);
  }
}
int64_t draw_dim() {
  static const int64_t dims[] = {16, 32, 64, 128, 256, 8, 48, 96, 0, -16, 512, I64MAX};
  return dims[next_u64() % (sizeof(dims) / sizeof(dims[0]))];
}

}  // namespace

namespace attn {
int launch(const Problem& pr, const LaunchArgs& a, void*) {
  ++g_calls;
  g_pr = pr;
  g_args = a;
  return g_launch_result;
}
}  // namespace attn

int main() {
  // ---- status strings
  for (int s = 0; s <= 5; ++s) {
    const char* t = attn_status_str((attn_status_t)s);
    EXPECT(t != nullptr && std::strcmp(t, "unknown status") != 0);
  }
  EXPECT(std::strcmp(attn_status_str((attn_status_t)99), "unknown status") == 0);
  EXPECT(std::strcmp(attn_status_str((attn_status_t)-1), "unknown status") == 0);
  EXPECT(attn_abi_version() == ATTN_ABI_VERSION);

  // ---- scalar checks (attn_fwd_check never launches)
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  EXPECT(attn_fwd_check(1, 1, 64, 128, nan, ATTN_MASK_NONE, 0, ATTN_F16) == ATTN_ERR_ARG);
  EXPECT(attn_fwd_check(1, 1, 64, 128, inf, ATTN_MASK_NONE, 0, ATTN_F16) == ATTN_ERR_ARG);
  EXPECT(attn_fwd_check(1, 1, 64, 128, -0.0f, ATTN_MASK_NONE, 0, ATTN_F16) == ATTN_ERR_ARG);
  EXPECT(attn_fwd_check(1, 1, 64, 128, 1e-45f, ATTN_MASK_NONE, 0, ATTN_F16) == ATTN_OK);
  EXPECT(attn_fwd_check(1, 1, 64, 128, 0.1f, (attn_mask_t)3, 0, ATTN_F16) == ATTN_ERR_ARG);
  EXPECT(attn_fwd_check(1, 1, 64, 128, 0.1f, ATTN_MASK_NONE, 0, (attn_dtype_t)4) == ATTN_ERR_ARG);
  EXPECT(attn_fwd_check(1, 1, 64, 128, 0.1f, (attn_mask_t)INT32_MIN, 0, ATTN_F16) == ATTN_ERR_ARG);
  // sizes at the int64 extremes
  const int64_t extremes[] = {I64MIN, I64MIN + 1, -1, 0, 1, INT32_MAX, (int64_t)1 << 31,
                              (int64_t)1 << 40, I64MAX - 1, I64MAX};
  for (int64_t a : extremes)
    for (int64_t b : extremes) {
      attn_status_t s = attn_fwd_check(a, b, 64, 128, 0.1f, ATTN_MASK_CAUSAL, 0, ATTN_BF16);
      EXPECT(s == ATTN_OK || s == ATTN_ERR_SHAPE);
      s = attn_fwd_check(1, a, b, 128, 0.1f, ATTN_MASK_NONE, 0, ATTN_F16);
      EXPECT(s == ATTN_OK || s == ATTN_ERR_SHAPE);
      s = attn_fwd_check(1, 1, a, b, 0.1f, ATTN_MASK_BLOCK_DIAG, 64, ATTN_F16);
      EXPECT(s == ATTN_OK || s == ATTN_ERR_SHAPE || s == ATTN_ERR_UNSUPPORTED);
      s = attn_fwd_check(1, 1, a, 128, 0.1f, ATTN_MASK_BLOCK_DIAG, b, ATTN_F16);
      EXPECT(s == ATTN_OK || s == ATTN_ERR_SHAPE || s == ATTN_ERR_UNSUPPORTED);
    }
  EXPECT(attn_fwd_check(1, 1, 256, 128, 0.1f, ATTN_MASK_BLOCK_DIAG, I64MIN, ATTN_F16) == ATTN_ERR_SHAPE);
  EXPECT(attn_fwd_check(1, 1, 256, 128, 0.1f, ATTN_MASK_BLOCK_DIAG, 100, ATTN_F16) == ATTN_ERR_SHAPE);
  EXPECT(attn_fwd_check(1, 1, 256, 128, 0.1f, ATTN_MASK_BLOCK_DIAG, 256, ATTN_F16) == ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_fwd_check(1, 1, 1 << 24, 128, 0.1f, ATTN_MASK_NONE, 0, ATTN_F16) == ATTN_ERR_SHAPE);

  // ---- contiguous entry points: accepted calls reach the launcher with the contiguous strides
  void* P = fake(0x100000);
  g_calls = 0;
  EXPECT(attn_fwd(P, P, P, P, 2, 3, 200, 128, 0.25f, ATTN_MASK_CAUSAL, 0, ATTN_BF16, nullptr) == ATTN_OK);
  EXPECT(g_calls == 1 && g_args.bh == 6 && g_args.heads == 3 && g_args.L == 200);
  EXPECT(g_args.lq.sb == 3 * 200 * 128 && g_args.lq.sh == 200 * 128 && g_args.lq.sr == 128);
  EXPECT(g_args.lse == nullptr && g_pr.mode == ATTN_MASK_CAUSAL && g_pr.dtype == ATTN_BF16);
  EXPECT(std::fabs(g_args.c - 0.25f * 1.44269504f) <= 1e-6f);
  float* lse = reinterpret_cast<float*>(fake(0x200004));
  EXPECT(attn_fwd_lse(P, P, P, P, lse, 1, 1, 64, 64, 0.125f, ATTN_MASK_NONE, 0, ATTN_F16, nullptr) == ATTN_OK);
  EXPECT(g_calls == 2 && g_args.lse == lse);
  // empty problems return OK without a launch; rejected ones never launch
  EXPECT(attn_fwd(P, P, P, P, 0, 3, 200, 128, 0.25f, ATTN_MASK_CAUSAL, 0, ATTN_BF16, nullptr) == ATTN_OK);
  EXPECT(attn_fwd(P, P, P, P, 2, 3, 0, 128, 0.25f, ATTN_MASK_BLOCK_DIAG, 64, ATTN_F16, nullptr) == ATTN_OK);
  EXPECT(attn_fwd(nullptr, P, P, P, 2, 3, 64, 128, 0.25f, ATTN_MASK_NONE, 0, ATTN_F16, nullptr) == ATTN_ERR_NULL);
  EXPECT(attn_fwd(P, P, P, P, 2, 3, 64, 96, 0.25f, ATTN_MASK_NONE, 0, ATTN_F16, nullptr) == ATTN_ERR_UNSUPPORTED);
  EXPECT(g_calls == 2);
  // a launch failure is reported as ATTN_ERR_HIP
  g_launch_result = 1;
  EXPECT(attn_fwd(P, P, P, P, 1, 1, 64, 64, 0.125f, ATTN_MASK_NONE, 0, ATTN_F16, nullptr) == ATTN_ERR_HIP);
  g_launch_result = 0;
  EXPECT(g_calls == 3);

  // ---- alignment: pointers and strides on 16-byte boundaries (lse on 4)
  const int64_t cont[3] = {2 * 64 * 128, 64 * 128, 128};
  g_calls = 0;
  for (uintptr_t off : {1u, 2u, 4u, 8u}) {
    void* M = fake(0x100000 + off);
    EXPECT(strided(M, P, P, P, nullptr, 1, 2, 64, 128, cont, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
    EXPECT(strided(P, M, P, P, nullptr, 1, 2, 64, 128, cont, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
    EXPECT(strided(P, P, M, P, nullptr, 1, 2, 64, 128, cont, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
    EXPECT(strided(P, P, P, M, nullptr, 1, 2, 64, 128, cont, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
    EXPECT(attn_fwd(M, P, P, P, 1, 2, 64, 128, 0.1f, ATTN_MASK_NONE, 0, ATTN_F16, nullptr) == ATTN_ERR_SHAPE);
  }
  float* bad_lse = reinterpret_cast<float*>(fake(0x200002));
  EXPECT(strided(P, P, P, P, bad_lse, 1, 2, 64, 128, cont, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
  const int64_t odd_head[3] = {2 * 64 * 128, 7, 128};           // 14 bytes
  const int64_t odd_row[3] = {2 * 64 * 136, 64 * 136, 132};     // 264 bytes per row
  const int64_t odd_batch[3] = {4, 64 * 128, 128};              // 8 bytes
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 128, odd_head, cont, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 128, cont, odd_row, cont, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 128, cont, cont, odd_batch, cont, 0.1f, 0, 0, 0) == ATTN_ERR_SHAPE);
  EXPECT(g_calls == 0);
  // fp8 V: one byte per element, so a row stride of 16 elements is one 16-byte unit; 8 is not
  const int64_t v8_ok[3] = {64 * 272, 0, 272};
  const int64_t v8_bad[3] = {64 * 264, 0, 264};
  const int64_t c256[3] = {2 * 64 * 256, 64 * 256, 256};
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 256, c256, c256, v8_ok, c256, 0.1f, 1, 0, 2) == ATTN_OK);
  EXPECT(g_calls == 1 && g_args.lv.sr == 272 && g_args.lv.sh == 0);
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 256, c256, c256, v8_bad, c256, 0.1f, 1, 0, 2) == ATTN_ERR_SHAPE);
  // the same strides for bf16 V are fine: 264 * 2 bytes is a multiple of 16
  EXPECT(strided(P, P, P, P, nullptr, 1, 2, 64, 256, c256, c256, v8_bad, c256, 0.1f, 1, 0, 1) == ATTN_OK);
  EXPECT(g_calls == 2);

  // ---- stride extremes: rejected, never launched, no undefined arithmetic
  g_calls = 0;
  const int64_t sx[] = {I64MIN, -16, 0, 8, 128, (int64_t)1 << 31, (int64_t)1 << 40, I64MAX / 2, I64MAX};
  for (int64_t a : sx)
    for (int64_t b : sx)
      for (int64_t c : {(int64_t)-128, (int64_t)128, (int64_t)4096, (int64_t)1 << 30, I64MAX}) {
        const int64_t st[3] = {a, b, c};
        const attn_status_t s =
            strided(P, P, P, P, nullptr, 3, 5, 100, 128, st, cont, cont, cont, 0.1f, 1, 0, 1);
        EXPECT(s == ATTN_OK || s == ATTN_ERR_SHAPE);
      }
  const int calls_extremes = g_calls;
  EXPECT(calls_extremes > 0);

  // ---- randomised: any mix of sizes, strides, pointers and enums
  long accepted = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    const int64_t B = draw_size(), H = draw_size(), L = draw_size(), D = draw_dim();
    int64_t st[4][3];
    for (auto& s : st)
      for (int64_t& x : s) x = (next_u64() % 3 == 0) ? draw_size() : 16 * (int64_t)(next_u64() % 100000);
    if (next_u64() % 2) {  // often a valid contiguous layout
      for (auto& s : st) {  // wrapping products: the sizes may be huge or negative here
        s[2] = D;
        s[1] = (int64_t)((uint64_t)L * (uint64_t)D);
        s[0] = (int64_t)((uint64_t)H * (uint64_t)s[1]);
      }
    }
    const int mode = (int)(next_u64() % 4);
    const int dt = (int)(next_u64() % 5);
    const int64_t bs = (next_u64() % 2) ? 64 : draw_size();
    const uintptr_t base = 0x100000 + ((next_u64() % 4 == 0) ? (next_u64() % 16) : 0);
    const float scale = (next_u64() % 8 == 0) ? -1.0f : 0.125f;
    const int before = g_calls;
    const attn_status_t s = strided(fake(base), P, P, P, nullptr, B, H, L, D, st[0], st[1], st[2],
                                    st[3], scale, mode, bs, dt);
    EXPECT(s >= ATTN_OK && s <= ATTN_ERR_ARG && s != ATTN_ERR_HIP);
    if (s == ATTN_OK) {
      ++accepted;
      const bool empty = B == 0 || H == 0 || L == 0;
      EXPECT(g_calls == before + (empty ? 0 : 1));
      if (!empty) EXPECT(g_args.bh == B * H && g_args.L == L && g_args.lq.sr == st[0][2]);
    } else {
      ++rejected;
      EXPECT(g_calls == before);
    }
    // attn_fwd_check agrees with the strided call on everything but the layout
    const attn_status_t c = attn_fwd_check(B, H, L, D, scale, (attn_mask_t)mode, bs, (attn_dtype_t)dt);
    EXPECT(c == ATTN_OK || s == c);
  }
  EXPECT(accepted > 1000 && rejected > 100000);
  std::printf("host checks passed: %ld checks, %ld random calls accepted, %ld rejected\n", g_checks,
              accepted, rejected);
  return 0;
}
