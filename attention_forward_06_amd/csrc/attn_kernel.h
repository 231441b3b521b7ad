// Attention forward kernels for gfx950, shared by the translation units that instantiate them:
// attn_fwd.hip (head dim 128 and block_diag) and attn_fwd_d256.hip (head dim 256, built with
// MFMA accumulators in VGPRs).  Head dims 16-64 (none and causal) run attn_fwd_rows64_kernel
// (attn_kernel_rows64.h), built on the helpers here.  Everything here has internal linkage, so
// each unit holds its own instances and the two sets never overlap.
//
// Fused scaled-dot-product attention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// One templated kernel covers the three mask modes:
//   none / causal  -- FlashAttention-2 online softmax over key tiles: running row max m,
//                     running exp-sum l, fp32 accumulator rescaled by alpha = 2^(m_old - m_new),
//                     O = acc / l at the end ("Triton-CUDA Attention", online-softmax core and
//                     full example; "Fused Attention", _attn_fwd_inner / _attn_fwd).  Causal
//                     runs the tiles left of the query block unmasked and masks only the
//                     tiles that straddle the diagonal ("Fused Attention", stages 1 and 2).
//   block_diag     -- one diagonal block per workgroup, a single key tile with an exact
//                     softmax and no rescaling ("TLX Block Attention", kernel).
// Exponentials are 2^x (v_exp_f32) with sm_scale * log2(e) folded into one FMA
// ("Triton-CUDA Attention", online-softmax core).
//
// gfx950 mapping (see the layout notes above each helper):
//   * Each wave owns 32 query rows.  It computes S^T = K_tile * Q^T with
//     v_mfma_f32_32x32x16_{f16,bf16}: K rows are the A operand (read from LDS), Q^T the
//     B operand (held in VGPRs for the whole loop).  The 32x32 accumulator then gives each
//     lane ONE query (lane % 32) and 16 of the tile's keys, so the row max / row sum are
//     in-lane plus one exchange with lane ^ 32.
//   * The K row fed to MFMA row rho is key pi(rho) (bits 2 and 3 of rho swapped).  With that
//     choice the 16 scores a lane holds per 32-key subtile are, per 16-key chunk, exactly the
//     8 consecutive keys the P.V MFMA wants from that lane -- P never leaves the registers.
//   * O^T = V^T * P^T: P^T is the B operand (the lane's own probabilities, packed to 16-bit or
//     fp8), V^T the A operand, read from the row-major V tile in LDS with the gfx950
//     transposing loads ds_read_b64_tr_b16 / ds_read_b64_tr_b8.  The O^T accumulator keeps
//     the lane's query too, so alpha and 1/l are per-lane scalars.
//   * fp8 V: P is rounded to OCP e5m2 (v_cvt_pk_bf8_f32, round-to-nearest-even) and P.V runs
//     on v_mfma_f32_32x32x64_f8f6f4 with both operands in bf8 (e5m2) format; the row sum uses
//     the unrounded fp32 P ("Fused Attention", _attn_fwd_inner fp8 branch).
//   * 16-bit P: the accumulator is rescaled only when a row max outgrows its reference by more
//     than 2^8, and O is normalised by the sum of the rounded weights P.V used (see Cfg).
//   * K/V tiles go HBM -> LDS by LDS-DMA (buffer_load ... lds, 16 bytes per lane, rows past L
//     read as zero), double-buffered with one barrier per tile; a software pipeline keeps K one
//     tile ahead of V so the score MFMAs of tile t+1 overlap the softmax of tile t.
//   * Any layout with a contiguous head dim (per-tensor batch / head / row strides); a head dim
//     of 16 (Cfg) runs head-dim-32 tiles with zero upper halves.
//   * Workgroup ids are remapped so all query blocks of one (batch, head) land on the same
//     XCD (its K/V stays in that XCD's L2); causal blocks run longest first within small head
//     groups, so the CUs of an XCD finish together.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn_host.h"

namespace {

typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
typedef unsigned int u32x2 __attribute__((__vector_size__(8)));
typedef int i32x8 __attribute__((__vector_size__(32)));
typedef int i32x2 __attribute__((__vector_size__(8)));
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef float f32x16 __attribute__((__vector_size__(64)));

constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskBlock = 2;
constexpr int kF16 = 0, kBF16 = 1, kBF16V8 = 2, kF16V8 = 3;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

using attn::Layout;

struct Params {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  unsigned char* o;
  float* lse;
  Layout lq, lk, lv, lo;
  int heads;
  int L;
  int bh;          // batch * heads
  int n_qblocks;   // query blocks per (batch, head)
  int group;       // causal: heads per longest-first group within an XCD (see block_coords)
  int tail;        // causal: the shortest query blocks, run by every XCD after all longer ones
  float c;         // sm_scale * log2(e)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// 128-bit load; offsets at or past the resource size return zeros.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == kF16) {
    f16x8 x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
  } else {
    bf16x8 x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
  }
}

// Two fp32 -> packed 16-bit (round to nearest even): one v_cvt_pk_{bf16,f16}_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (DT == kF16) return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
  else return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// acc + (lo + hi) of a packed 16-bit pair (v_dot2 against (1, 1)).
template <int DT>
__device__ __forceinline__ float sum2_acc(unsigned packed, float acc) {
  if constexpr (DT == kF16) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
  } else {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
  }
}

// MFMA row rho of the S^T = K * Q^T product reads key pi(rho): bits 2 and 3 swapped.
__device__ __forceinline__ int key_of_row(int rho) {
  return (rho & 0x13) | ((rho & 4) << 1) | ((rho >> 1) & 4);
}


template <int D, int DT, int MODE, int NW, int BN, int KW = BN>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * NW;
  // KW: keys one wave works on per tile.  KW = BN except for block_diag with blocks smaller
  // than the tile, where each wave only touches its own diagonal block inside the tile.
  static constexpr int KT = KW / 32;          // 32-key subtiles a wave computes per tile
  // Tile head dim: D = 16 runs as 32, with the upper half of every Q, K and V row zero (the DMA
  // and the Q loads fill it with zeros; the epilogue stores only d < D).
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int DK = DP / 16;          // 16-wide d chunks of Q.K
  static constexpr int DTL = DP / 32;         // 32-wide d tiles of O
  static constexpr bool V8 = (DT == kBF16V8 || DT == kF16V8);
  static constexpr int QK = (DT == kF16 || DT == kF16V8) ? kF16 : kBF16;   // Q, K and O element type
  static constexpr int VB = V8 ? 1 : 2;       // bytes per V element
  static constexpr int KROWB = DP * 2;        // bytes per K row in LDS (no padding: XOR swizzle)
  static constexpr int VROWB = DP * VB;       // bytes per V row in LDS
  static constexpr int KGROWB = D * 2;        // bytes per K row in HBM
  static constexpr int VGROWB = D * VB;       // bytes per V row in HBM
  static constexpr int KTILE = BN * KROWB;
  static constexpr int VTILE = BN * VROWB;
  static constexpr int NBUF = MODE == kMaskBlock ? 1 : 2;   // double-buffer the streamed tiles
  static constexpr int KDMA = KTILE / 1024 / NW;  // 1 KiB LDS-DMA instructions per wave per K tile
  static constexpr int VDMA = VTILE / 1024 / NW;
  // Period (in DMA instruction index i) of a lane's swizzled offset: instruction i starts
  // i * NW * 1024 / ROWB rows further on, and the swizzles only read the row modulo
  // 16 (K), 8 (fp8 V) or 4 (16-bit V).
  static constexpr int period(int rows_per_step, int modulus) {
    int p = 1;
    while ((p * rows_per_step) % modulus != 0) ++p;
    return p;
  }
  static constexpr int KPER = period(NW * 1024 / KROWB, 16);
  static constexpr int VPER = period(NW * 1024 / VROWB, V8 ? 8 : 4);
  // The accumulator is rescaled when a row max grows by more than 2^TAU over the reference it
  // was accumulated against (exact in real arithmetic: O = acc / l in a common frame); a wave
  // skips the rescale when no row of it needs one.  The fp8 path uses TAU = 0, the pages'
  // recurrence, so P is rounded against the running maximum exactly as the pages do.
  static constexpr float TAU = V8 ? 0.f : 8.f;
  // 16-bit P: O is normalised by the sum of the rounded weights P^ that P.V actually used.
  // O = sum P^ v / sum P^ is then an exactly normalised average of the V rows -- exact for a
  // single dominant key and for constant V -- which is what makes the capped rescale above safe.
  // The fp8 path keeps the pages' sum over the unrounded p (P is far coarser there).
  static constexpr bool HAT = !V8;
  static constexpr int WAVES_PER_EU = (D >= 256) ? 1 : 2;
  // General (compiler-scheduled) iteration with two waves on a SIMD: the wave in its MFMA
  // stretch (S(t+1), the exponentials of P(t), P(t).V(t)) is raised above the other, which is
  // then in its barrier / DMA / row-max stretch, so the matrix core gets the shared issue port
  // first.  The explicit unmasked streams mix both stretches in every wave and leave the
  // priority alone.  With one wave per SIMD there is no rival.
  static constexpr bool PRIO = WAVES_PER_EU > 1;
  static_assert(BN % 32 == 0, "key tile is a whole number of 32-key subtiles");
  static_assert(!V8 || BN % 64 == 0, "fp8 P.V consumes 64 keys per MFMA");
  static_assert(KTILE % (1024 * NW) == 0 && VTILE % (1024 * NW) == 0,
                "tiles split into whole 1 KiB DMA instructions per wave");
  static_assert(DP % 32 == 0 && (D == DP || D == 16), "head dim 16 or a multiple of 32");
};

// XOR swizzles of the 16-byte chunks inside a tile row (LDS-DMA writes rows unpadded).
// K: the 16 lanes of a ds_read_b128 read the same chunk of 16 different rows (rows 0..15 up to
//    the bit swap pi) -> spread them over 16 distinct chunk positions of a 256-byte bank window:
//    a row of ROWB bytes holds ROWB/16 chunks, 256/ROWB rows share a window, and the XOR takes
//    the row bits above those.
// V (16-bit): a ds_read_b64_tr_b16 half-wave reads 4 rows x 64 contiguous bytes -> give the
//    4 rows disjoint 64-byte slots (64-byte rows already are).   V (fp8): tr_b8 reads 8 rows x
//    32 bytes -> 8 slots of 32.
template <int ROWB>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (ROWB == 64) return (r >> 2) & 3;
  else if constexpr (ROWB == 128) return (r >> 1) & 7;
  else return r & 15;
}
template <int ROWB, bool V8>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (V8) return 2 * (r & 7);
  else if constexpr (ROWB == 64) return 0;
  else if constexpr (ROWB == 128) return 4 * ((r >> 1) & 1);
  else return 4 * (r & 3);
}

// Workgroup id -> (batch*head, query block).  Ids are dealt round-robin to the 8 XCDs; the remap
// gives each XCD a contiguous range of heads, so one head's K/V is shared in one L2.  Causal query
// blocks differ in length (block qb walks qb + 1 key blocks), so an XCD runs its heads in groups
// of `group`, all query blocks of a group longest first: the blocks that start last are short
// and the XCD's CUs finish together.  The host sizes the group so that its K/V fits the L2.
// With `tail` > 0 the `tail` shortest blocks of every head are held back and run after all other
// blocks of the XCD, longest first across its heads: otherwise the last group's longest blocks
// start late and leave CUs idle at the end.
__device__ __forceinline__ void block_coords(int id, int total, int nqb, bool heavy_first, int group,
                                             int tail, int& bh, int& qb) {
  const int per_xcd = total >> 3;
  if ((total & 7) == 0 && heavy_first && per_xcd % (nqb * group) == 0 && tail < nqb) {
    const int x = id & 7, j = id >> 3;
    const int hx = per_xcd / nqb, nl = nqb - tail;   // heads of this XCD, blocks run in groups
    if (j < hx * nl) {
      const int g = j / (group * nl), r = j - g * (group * nl);
      qb = nqb - 1 - r / group;
      bh = x * hx + g * group + r % group;
    } else {
      const int j2 = j - hx * nl;
      qb = tail - 1 - j2 / hx;
      bh = x * hx + j2 % hx;
    }
    return;
  }
  int logical = id;
  if ((total & 7) == 0) logical = (id & 7) * per_xcd + (id >> 3);
  bh = logical / nqb;
  qb = logical - bh * nqb;
  if (heavy_first) qb = nqb - 1 - qb;
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// Value of the lane 32 places away (lanes l and l^32 hold the two halves of one query row).
__device__ __forceinline__ float partner(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  // r[0]: lanes 32..63 received lanes 0..31; r[1]: lanes 0..31 received lanes 32..63
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// One tile of K or V, HBM -> LDS by DMA (see the kernel for the layout).  A device function:
// the same code written as a lambda inside the kernel made the host compiler drop the kernel's
// launch stub.
// inside: the caller knows the whole tile lies below row L (no per-row check).
// rs: bytes between consecutive rows in HBM.
template <int ROWB, int NI, int PER, int NW, int BN>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, int key0, int L, int rs, int wave,
                                         int lane, unsigned oob, const unsigned* off, unsigned char* buf,
                                         const bool inside) {
  constexpr int RPI = NW * 1024 / ROWB;              // tile rows one instruction index covers
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    auto* dst = (__attribute__((address_space(3))) void*)(buf + (wave + i * NW) * 1024);
    // Scalar part of the offset, made opaque (readfirstlane of a uniform value): otherwise the
    // compiler splits off each index's constant row offset times the run-time row stride and
    // adds it to the lane offset in a separate register per index, held through the loop.
    const int soff = __builtin_amdgcn_readfirstlane((key0 + i * RPI) * rs);
    const unsigned vo = off[i % PER];
    if (inside) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, vo, soff, 0, 0);
    } else {
      // the tile's first key through an empty asm: keeps the compiler from computing these
      // per-lane checks ahead of the scalar branch that selects this (rarely taken) path
      int k0 = key0;
      asm volatile("" : "+s"(k0));
      const int row = ((wave + i * NW) * 1024 + lane * 16) / ROWB;
      const unsigned o = k0 + row < L ? vo + (unsigned)soff : oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, o, 0, 0, 0);
    }
  }
}

template <int D, int DT, int MODE, int NW, int BN, int KW, bool LSE>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(Cfg<D, DT, MODE, NW, BN, KW>::WAVES_PER_EU)))
void attn_fwd_kernel(Params p) {
  using C = Cfg<D, DT, MODE, NW, BN, KW>;
  // One statically sized LDS array per tile buffer, so the compiler can tell the buffer being
  // read from the one the DMA is filling (it then does not wait for that DMA before reading).
  __shared__ __attribute__((aligned(1024))) unsigned char lk0[C::KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char lv0[C::VTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char lk1[C::NBUF == 2 ? C::KTILE : 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char lv1[C::NBUF == 2 ? C::VTILE : 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int h = lane >> 5;        // which half of the wave (k sub-block of the MFMA operands)
  const int col = lane & 31;      // the lane's query within the wave's 32

  int bh, qb;
  block_coords(blockIdx.x, gridDim.x, p.n_qblocks, MODE == kMaskCausal, p.group, p.tail, bh, qb);
  const int L = p.L;
  const int m0 = qb * C::BM;              // first query row of the workgroup
  const int qw0 = m0 + 32 * wave;         // first query row of this wave
  const int my_q = qw0 + col;

  // This head's rows of each tensor: base, row stride, and extent (the buffer resources end at the
  // last row, so rows at or past L -- and the padding offset -- read as zeros).
  const int bi = bh / p.heads, hi = bh - bi * p.heads;
  const unsigned char* qh = p.q + (size_t)(bi * p.lq.sb + hi * p.lq.sh) * 2;
  const unsigned char* kh = p.k + (size_t)(bi * p.lk.sb + hi * p.lk.sh) * 2;
  const unsigned char* vh = p.v + (size_t)(bi * p.lv.sb + hi * p.lv.sh) * C::VB;
  const int q_rs = p.lq.sr * 2, k_rs = p.lk.sr * 2, v_rs = p.lv.sr * C::VB;   // bytes per row
  const unsigned q_ext = (unsigned)((L - 1) * q_rs + D * 2);
  const unsigned k_oob = (unsigned)((L - 1) * k_rs + D * 2);
  const unsigned v_oob = (unsigned)((L - 1) * v_rs + D * C::VB);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, q_ext);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, k_oob);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, v_oob);

  // HBM -> LDS by DMA: instruction j of a tile fills LDS bytes [1024 j, 1024 j + 1024); lane l
  // lands at +16 l.  The lane fetches the global chunk that the swizzle stores at that slot.
  // Per lane the row within the instruction's block of rows and the chunk are fixed; instruction
  // index i and the tile add (key0 + i * rows per index) * row_bytes as a scalar offset.  Tiles
  // reaching past row L take the checked path, where rows at or past L read as zeros; so do the
  // chunks of a padded row (D = 16), whose offset is past any buffer.
  // The lane's chunk repeats with period KPER (VPER) in i: the swizzle only looks at low row bits.
  constexpr unsigned kPadOff = 0x80000000u;
  unsigned k_off[C::KPER], v_off[C::VPER];
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) {
    const int byte = (wave + i * NW) * 1024 + lane * 16;
    const int row = byte / C::KROWB;
    const int lch = ((byte % C::KROWB) >> 4) ^ swz_k<C::KROWB>(row);   // chunk stored at this slot
    const int rin = (wave * 1024 + lane * 16) / C::KROWB;               // row - i * rows per index
    k_off[i] = lch * 16 < C::KGROWB ? (unsigned)(rin * k_rs + lch * 16) : kPadOff;
  }
#pragma unroll
  for (int i = 0; i < C::VPER; ++i) {
    const int byte = (wave + i * NW) * 1024 + lane * 16;
    const int row = byte / C::VROWB;
    const int lch = ((byte % C::VROWB) >> 4) ^ swz_v<C::VROWB, C::V8>(row);
    const int rin = (wave * 1024 + lane * 16) / C::VROWB;
    v_off[i] = lch * 16 < C::VGROWB ? (unsigned)(rin * v_rs + lch * 16) : kPadOff;
  }
  // One scalar branch per tile selects the unchecked copy when no row of the tile is past L.
  auto dma_k = [&](int key0, unsigned char* kb) __attribute__((always_inline)) {
    if (key0 + BN <= L) dma_rows<C::KROWB, C::KDMA, C::KPER, NW, BN>(rk, key0, L, k_rs, wave, lane, k_oob, k_off, kb, true);
    else dma_rows<C::KROWB, C::KDMA, C::KPER, NW, BN>(rk, key0, L, k_rs, wave, lane, k_oob, k_off, kb, false);
  };
  auto dma_v = [&](int key0, unsigned char* vb) __attribute__((always_inline)) {
    if (key0 + BN <= L) dma_rows<C::VROWB, C::VDMA, C::VPER, NW, BN>(rv, key0, L, v_rs, wave, lane, v_oob, v_off, vb, true);
    else dma_rows<C::VROWB, C::VDMA, C::VPER, NW, BN>(rv, key0, L, v_rs, wave, lane, v_oob, v_off, vb, false);
  };

  // Key range walked by this workgroup.
  int key_begin = 0, key_end = L;
  if constexpr (MODE == kMaskCausal) key_end = min(L, m0 + C::BM);
  if constexpr (MODE == kMaskBlock) {
    key_begin = m0;
    key_end = m0 + C::BM;
  }
  const int ntiles = (key_end - key_begin + BN - 1) / BN;

  // Software pipeline: iteration t computes the scores of tile t+1 on MFMA while the VALU runs
  // the softmax of tile t, then P.V of tile t.  K therefore streams one tile ahead of V:
  // tile j's K and V both live in buffer j % 2; at the top of iteration t (after the barrier)
  // the DMA fills K(t+2) into the K buffer tile t used and V(t+1) into the V buffer of t-1.
  if (ntiles > 0) {
    dma_k(key_begin, lk0);
    dma_v(key_begin, lv0);
  }
  if (ntiles > 1) dma_k(key_begin + BN, lk1);

  // Q^T fragment (B operand): lane holds Q[my_q][16*kk + 8*h .. +7] for every kk.
  u32x4 qf[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    const bool in = my_q < L && 16 * kk + 8 * h < D;   // d >= D: the zero half of a padded row
    const unsigned off = in ? (unsigned)(my_q * q_rs + (16 * kk + 8 * h) * 2) : q_ext;
    qf[kk] = buf_load16(rq, off);
  }

  f32x16 acc[C::DTL];
#pragma unroll
  for (int dt = 0; dt < C::DTL; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_ref = -INFINITY;   // reference max (scores * c, log2 domain) acc and l are relative to
  float l_run = 0.f;         // running sum of 2^(s*c - m_ref) over this lane's keys (unrounded)
  float l_hat = 0.f;         // the same over the rounded 16-bit weights (16-bit P only)

  // block_diag with blocks smaller than the tile: this wave's block is rows [wrow, wrow + KW)
  // of the tile (the workgroup's 128 rows hold 128 / KW diagonal blocks, wave-aligned).
  const int wrow = (MODE == kMaskBlock && KW < BN) ? (32 * wave / KW) * KW : 0;
  // Per-lane LDS offsets that do not change across tiles.
  const int krow = key_of_row(col) + wrow;                // + 32*kt for subtile kt
  const int kswz = swz_k<C::KROWB>(krow);                 // same for krow + 32*kt
  const int k_lane_off = krow * C::KROWB;
  // ds_read_b64_tr_b16: in each 16-lane group, lane 4e+q supplies the address of row e,
  // 4-element column block q; the instruction hands lane 4q+c element e of that block.
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr16_row = 8 * (g16 >> 1) + (s16 >> 2) + wrow;  // + 16*cc + 4*t
  const int tr16_cb = 32 * (g16 & 1) + 8 * (s16 & 3);      // byte in a 64-byte d tile
  // ds_read_b64_tr_b8: lane 2e+q supplies row e, 8-byte column block q.
  const int tr8_row = 8 * (g16 >> 1) + (s16 >> 1) + wrow;  // + 64*u64 + 16*t4
  const int tr8_cb = 16 * (g16 & 1) + 8 * (s16 & 1);      // byte in a 32-byte d tile

  // Tiles [0, nfull) are visible to every query row of the workgroup (no liveness test, no
  // mask); the causal diagonal and a ragged tail take the general path.
  int nfull = ntiles;
  if constexpr (MODE == kMaskCausal) nfull = min(ntiles, (m0 + 1) / BN);
  if constexpr (MODE == kMaskNone) nfull = min(ntiles, L / BN);


  // Which 32-key subtiles of tile j this wave needs, and which need an element mask.
  auto tile_flags = [&](int j, const bool FULL, bool* live, bool* masked) __attribute__((always_inline)) {
    const int key0 = key_begin + j * BN;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      const int n0 = key0 + 32 * kt;
      if (FULL) {
        live[kt] = true;
        masked[kt] = false;
      } else if constexpr (MODE == kMaskCausal) {
        live[kt] = n0 <= qw0 + 31;
        masked[kt] = n0 + 31 > qw0;
      } else if constexpr (MODE == kMaskNone) {
        live[kt] = n0 < L;
        masked[kt] = n0 + 31 >= L;
      } else {
        live[kt] = true;
        masked[kt] = false;
      }
    }
  };

  // S^T = K * Q^T for the live subtiles of one tile, in two parts so that all K fragment reads
  // can be issued well before the MFMAs that consume them.
  // ksw: the lane's K swizzle (kswz); the masked iterations pass an opaque copy so that their
  // read addresses are recomputed instead of being held in registers across the loops.
  auto k_frags = [&](u32x4 (*fr)[C::DK], const unsigned char* kbuf, const bool* live, int ksw) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < (D <= 128 ? 1 : 0); ++kt)
      if (live[kt]) {
        const unsigned char* kb = kbuf + k_lane_off + 32 * kt * C::KROWB;
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) fr[kt][kk] = *(const u32x4*)(kb + (((2 * kk + h) ^ ksw) << 4));
      }
  };
  auto scores = [&](f32x16* s, u32x4 (*fr)[C::DK], const unsigned char* kbuf, const bool* live, int ksw) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      if (!live[kt]) continue;
      f32x16 z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        u32x4 a;
        if (D <= 128 && kt == 0) a = fr[kt][kk];
        else a = *(const u32x4*)(kbuf + k_lane_off + 32 * kt * C::KROWB + (((2 * kk + h) ^ ksw) << 4));
        z = mfma_qk<C::QK>(a, qf[kk], z);
      }
      s[kt] = z;
    }
  };

  // Mask, online-softmax update and O += P.V for tile t whose scores are in s.
  auto softmax_max = [&](int t, f32x16* s, const bool* live, const bool* masked) __attribute__((always_inline)) {
    const int key0 = key_begin + t * BN;
    // ---- mask, row max ------------------------------------------------------------------
    // Lane's register r of subtile kt holds key key0 + 32*kt + 16*(r/8) + 8*h + r%8.
    // One max3 chain per 32-key subtile.  The empty asm makes each step opaque: left alone, the
    // compiler rebalances a chain into pairwise maxima plus a shorter max3 chain, 24 instructions
    // per 64 keys instead of 18.
    float mk[C::KT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      mk[kt] = -INFINITY;
      if (!live[kt]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = -INFINITY;
        continue;
      }
      if (masked[kt]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kt + 16 * (r >> 3) + 8 * h + (r & 7);
          bool ok;
          if constexpr (MODE == kMaskCausal) ok = key <= my_q;
          else ok = key < L;
          if (!ok) s[kt][r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        mk[kt] = max3(mk[kt], s[kt][r], s[kt][r + 1]);
        asm("" : "+v"(mk[kt]));
      }
    }
    float mx = mk[0];
#pragma unroll
    for (int kt = 1; kt < C::KT; ++kt) mx = __builtin_fmaxf(mx, mk[kt]);
    mx = __builtin_fmaxf(mx, partner(mx));

    // ---- online softmax update ------------------------------------------------------------
    const float m_cand = mx * p.c;
    if constexpr (MODE == kMaskBlock) {
      m_ref = m_cand;                              // single tile: exact max, nothing to rescale
    } else {
      const bool need = m_cand > m_ref + C::TAU;   // always true on a lane's first live tile
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? m_cand : m_ref;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;  // 0 at first
        m_ref = m_new;
        l_run *= alpha;
        l_hat *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DTL; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      }
    }
  };
  // P = 2^(s c - m_ref).  16-bit: packed right away into pk (the P.V operand) with the sum of
  // the rounded pairs; the unrounded sum only when the log-normaliser is requested.
  auto softmax_exp = [&](f32x16* s, u32x4* pk, const bool* live) __attribute__((always_inline)) {
    const float neg = -m_ref;
    if constexpr (C::HAT) {
      float lh = 0.f, le = 0.f;
#pragma unroll
      for (int cc = 0; cc < KW / 16; ++cc) {
        const int kt = cc >> 1, c8 = (cc & 1) * 8;
        if (!live[kt]) continue;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][c8 + 2 * w], p.c, neg));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][c8 + 2 * w + 1], p.c, neg));
          pk[cc][w] = pack2<DT>(e0, e1);
          lh = sum2_acc<DT>(pk[cc][w], lh);
          if constexpr (LSE) le += e0 + e1;
        }
      }
      l_hat += lh;
      if constexpr (LSE) l_run += le;
    } else {
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], p.c, neg));
          s[kt][r] = e;
          psum += e;
        }
      l_run += psum;
    }
  };
  auto pv = [&](f32x16* s, const u32x4* pk, const unsigned char* vbuf, const bool* live) __attribute__((always_inline)) {
    // ---- O^T += V^T * P^T -----------------------------------------------------------------
    if constexpr (!C::V8) {
#pragma unroll
      for (int cc = 0; cc < KW / 16; ++cc) {
        const int kt = cc >> 1;
        if (!live[kt]) continue;
        const u32x4 pb = pk[cc];
#pragma unroll
        for (int dt = 0; dt < C::DTL; ++dt) {
          u32x4 a;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int row = 16 * cc + 4 * tt + tr16_row;
            const int byte = 64 * dt + tr16_cb;
            const int sw = ((byte >> 4) ^ swz_v<C::VROWB, false>(row)) << 4 | (byte & 15);
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vbuf + row * C::VROWB + sw));
            __builtin_memcpy((char*)&a + 8 * tt, &x, 8);
          }
          acc[dt] = mfma_qk<DT>(a, pb, acc[dt]);
        }
      }
    } else {
#pragma unroll
      for (int u64 = 0; u64 < KW / 64; ++u64) {
        if (!live[2 * u64] && !live[2 * u64 + 1]) continue;
        // P bytes: byte 16*u + r <- subtile 2*u64+u, register r (key 16*(2u + r/8) + 8h + r%8).
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int u = w >> 2, r = (w & 3) * 4;
          int word = __builtin_amdgcn_cvt_pk_bf8_f32(s[2 * u64 + u][r], s[2 * u64 + u][r + 1], 0, false);
          word = __builtin_amdgcn_cvt_pk_bf8_f32(s[2 * u64 + u][r + 2], s[2 * u64 + u][r + 3], word, true);
          pb[w] = word;
        }
#pragma unroll
        for (int dt = 0; dt < C::DTL; ++dt) {
          i32x8 a;
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) {
            const int row = 64 * u64 + 16 * t4 + tr8_row;
            const int byte = 32 * dt + tr8_cb;
            const int sw = ((byte >> 4) ^ swz_v<C::VROWB, true>(row)) << 4 | (byte & 15);
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(vbuf + row * C::VROWB + sw));
            a[2 * t4] = x[0];
            a[2 * t4 + 1] = x[1];
          }
          acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, acc[dt], 1, 1, 0, 0, 0, 0);
        }
      }
    }
  };

  // One pipelined iteration; buffers are passed in so that the unrolled copies see fixed ones.
  // fast: tiles t and t+1 are both unmasked (a constant at every call).
  auto iteration = [&](const bool fast, int t, f32x16* s_cur, f32x16* s_nxt,
                       const unsigned char* kb_nxt, const unsigned char* vb_cur, unsigned char* kb_dma,
                       unsigned char* vb_dma) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA of K(t+1), V(t) landed
    __syncthreads();                 // everyone's did; nobody still reads K(t) or V(t-1)
    if (t + 2 < ntiles) dma_k(key_begin + (t + 2) * BN, kb_dma);
    if (t + 1 < ntiles) dma_v(key_begin + (t + 1) * BN, vb_dma);
    const bool has_next = t + 1 < ntiles;
    int ksw = kswz;
    if (!fast) asm volatile("" : "+v"(ksw));
    bool live_n[C::KT], masked_n[C::KT];
    u32x4 fr[C::KT][C::DK];
    if (has_next) {
      tile_flags(t + 1, fast || t + 1 < nfull, live_n, masked_n);
      k_frags(fr, kb_nxt, live_n, ksw);        // K(t+1) reads, in flight during the max below
    }
    bool live[C::KT], masked[C::KT];
    tile_flags(t, fast || t < nfull, live, masked);
    softmax_max(t, s_cur, live, masked);       // VALU: mask, row max, rescale
    if constexpr (C::PRIO) __builtin_amdgcn_s_setprio(1);
    if (has_next) scores(s_nxt, fr, kb_nxt, live_n, ksw);   // MFMA: S(t+1) ...
    u32x4 pk[KW / 16];
    softmax_exp(s_cur, pk, live);              // ... while the VALU exponentiates P(t)
    pv(s_cur, pk, vb_cur, live);               // MFMA: O += P(t) V(t)
    if constexpr (C::PRIO) __builtin_amdgcn_s_setprio(0);
    if constexpr (D <= 128 && C::KT == 2 && !C::V8 && MODE != kMaskBlock) {
      if (fast && has_next) {
        // Issue order of the unmasked iteration: each score MFMA of subtile 0 followed by one K
        // read of subtile 1, each of subtile 1 by two V^T reads, each P.V MFMA by one more V^T
        // read, with the exponentials spread over the score MFMAs.  Every LDS read is then
        // issued several MFMAs ahead of its use.
        constexpr int NP = (KW / 16) * C::DTL, NV_LATE = 2 * NP - 2 * C::DK;
        static_assert(NV_LATE == NP, "one late V^T read per P.V MFMA");
        constexpr int VS = 32 / C::DK, VP = 32 / NP;
#pragma unroll
        for (int i = 0; i < C::DK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VS, 0);
        }
#pragma unroll
        for (int i = 0; i < C::DK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VS, 0);
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VP, 0);
        }
      }
    }
    if constexpr (D == 256 && MODE != kMaskBlock) {
      if (fast && has_next) {
        // D = 256 runs one wave per SIMD, so nothing hides an LDS read issued right before its
        // MFMA.  Issue order: four K reads, then one K read after each score MFMA (reads stay
        // four MFMAs ahead), half of the V^T reads after the last four score MFMAs and the rest
        // after the first P.V MFMAs, with the exponentials spread over the score MFMAs.
        constexpr int NS = C::KT * C::DK;
        constexpr int RPP = C::V8 ? 4 : 2;                          // V^T reads per P.V MFMA
        constexpr int NP = C::V8 ? (KW / 64) * C::DTL : (KW / 16) * C::DTL;
        constexpr int NV = NP * RPP, NVE = NV / 2, KA = 4;
        static_assert(NVE % KA == 0 && (NV - NVE) % RPP == 0, "V^T reads split evenly");
        __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);
#pragma unroll
        for (int i = 0; i < NS - KA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
#pragma unroll
        for (int i = 0; i < KA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, NVE / KA, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
#pragma unroll
        for (int i = 0; i < (NV - NVE) / RPP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, RPP, 0);
        }
      }
    }
  };

  // Capped rescale of the accumulator to a row max m_cand (scores * c) already taken.
  auto rescale_to = [&](float m_cand) __attribute__((always_inline)) {
    const bool need = m_cand > m_ref + C::TAU;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? m_cand : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      l_run *= alpha;
      l_hat *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DTL; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
  };

  // Unmasked iteration at head dims 128 and 256 with 16-bit P, written as an explicit issue
  // stream.
  // Each group is one MFMA, the LDS reads of operands several MFMAs ahead, and a slice of VALU
  // work; a scheduling barrier closes each group, so the order below is the order issued.
  //   * score MFMA i (subtile i / DK, chunk i % DK) reads K fragment i, read NKA MFMAs ahead;
  //     the P.V MFMAs read V^T fragments NVA MFMAs ahead, the first ones during the last score
  //     MFMAs;
  //   * the exponentials of P(t) -- 16 pair-items (chunk cc, pair w: two FMAs, two
  //     exponentials, one pack, one pair sum) -- are spread evenly over the score MFMAs of S(t+1)
  //     (one per MFMA at D = 128, one every second MFMA at D = 256), pipelined one item deep
  //     (exponentials of item k, pack and sum of item k - 1);
  //   * the row max of S(t+1) is spread over the P.V MFMAs (subtile 0 in the first half;
  //     subtile 1, whose last score MFMA is still running when P.V starts, in the second), and
  //     the reference moves (rarely) after them, so the next iteration starts with its
  //     exponentials.  The loop prologue takes the row max of tile 0.
  // A/B on one GPU against the compiler-scheduled iteration: +2% causal and +3% unmasked at
  // D = 128; +31% causal and +16% unmasked at D = 256 (one wave per SIMD: nothing else hides a
  // late operand there).
  constexpr bool EXPL = (D == 128 || D == 256) && !C::V8 && MODE != kMaskBlock && C::KT == 2;
  auto fast_iter_expl = [&](int t, f32x16* s_cur, f32x16* s_nxt, const unsigned char* kb_nxt,
                            const unsigned char* vb_cur, unsigned char* kb_dma, unsigned char* vb_dma) __attribute__((always_inline)) {
    constexpr int NSM = 2 * C::DK;            // score MFMAs
    constexpr int NPM = (BN / 16) * C::DTL;   // P.V MFMAs
    constexpr int NKA = 6;                    // K fragments read ahead
    constexpr int NVA = 4;                    // V^T fragments read ahead
    constexpr int NIT = (BN / 16) * 4;        // exponential pair-items
    constexpr int NMX = 8;                    // max3 steps per 32-key subtile
    static_assert(!EXPL || (NSM % NIT == 0 && NPM % 2 == 0 && NKA >= NVA), "issue stream shape");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < ntiles) dma_k(key_begin + (t + 2) * BN, kb_dma);
    if (t + 1 < ntiles) dma_v(key_begin + (t + 1) * BN, vb_dma);
    auto kread = [&](int i) __attribute__((always_inline)) {
      const int kt = i / C::DK, kk = i % C::DK;
      return *(const u32x4*)(kb_nxt + k_lane_off + 32 * kt * C::KROWB + (((2 * kk + h) ^ kswz) << 4));
    };
    auto vread = [&](int j) __attribute__((always_inline)) {
      const int cc = j / C::DTL, dt = j % C::DTL;
      u32x4 a;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 16 * cc + 4 * tt + tr16_row;
        const int byte = 64 * dt + tr16_cb;
        const int sw = ((byte >> 4) ^ swz_v<C::VROWB, false>(row)) << 4 | (byte & 15);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vb_cur + row * C::VROWB + sw));
        __builtin_memcpy((char*)&a + 8 * tt, &x, 8);
      }
      return a;
    };
    u32x4 kf[NSM], vf[NPM];
#pragma unroll
    for (int i = 0; i < NKA; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
    const float neg = -m_ref;
    u32x4 pk[BN / 16];
    float lh = 0.f, le = 0.f;
    float e0[NIT], e1[NIT];
    auto item_exp = [&](int k) __attribute__((always_inline)) {
      const int cc = k >> 2, w = k & 3, kt = cc >> 1, c8 = (cc & 1) * 8;
      e0[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kt][c8 + 2 * w], p.c, neg));
      e1[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kt][c8 + 2 * w + 1], p.c, neg));
    };
    auto item_pack = [&](int k) __attribute__((always_inline)) {
      const int cc = k >> 2, w = k & 3;
      pk[cc][w] = pack2<DT>(e0[k], e1[k]);
      lh = sum2_acc<DT>(pk[cc][w], lh);
      if constexpr (LSE) le += e0[k] + e1[k];
    };
    f32x16 z0, z1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z0[r] = 0.f;
      z1[r] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NSM; ++i) {
      if (i < C::DK) z0 = mfma_qk<C::QK>(kf[i], qf[i % C::DK], z0);
      else z1 = mfma_qk<C::QK>(kf[i], qf[i % C::DK], z1);
      const int j = i + NKA;
      if (j < NSM) kf[j] = kread(j);
      else if (j - NSM < NPM) vf[j - NSM] = vread(j - NSM);
      // item k rides on score MFMA (k * NSM) / NIT
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        if ((k * NSM) / NIT != i) continue;
        item_exp(k);
        if (k > 0) item_pack(k - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    item_pack(NIT - 1);
    s_nxt[0] = z0;
    s_nxt[1] = z1;
    l_hat += lh;
    if constexpr (LSE) l_run += le;
    __builtin_amdgcn_sched_barrier(0);
    float mk[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int j = 0; j < NPM; ++j) {
      const int cc = j / C::DTL, dt = j % C::DTL;
      acc[dt] = mfma_qk<DT>(vf[j], pk[cc], acc[dt]);
      const int jn = j + NKA;
      if (jn < NPM) vf[jn] = vread(jn);
#pragma unroll
      for (int q = 0; q < 2 * NMX; ++q) {
        const int kt = q / NMX, r = 2 * (q % NMX);
        if (kt * (NPM / 2) + ((q % NMX) * (NPM / 2)) / NMX != j) continue;
        mk[kt] = max3(mk[kt], s_nxt[kt][r], s_nxt[kt][r + 1]);
        asm("" : "+v"(mk[kt]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float mx = __builtin_fmaxf(mk[0], mk[1]);
    mx = __builtin_fmaxf(mx, partner(mx));
    rescale_to(mx * p.c);
  };

  // Unmasked iteration at head dim 256 with e5m2 V, as an explicit issue stream (one wave per
  // SIMD: nothing else hides a late operand).  Score MFMA i (subtile i / DK, chunk i % DK) reads
  // K fragment i, read NKA MFMAs ahead.  Each score MFMA carries one weight of P(t) (FMA,
  // exponential, unrounded row sum); every fourth packs four weights to e5m2 (the P operand of
  // the fp8 MFMAs), so the fp32 scores of S(t) are released as the pass goes.  The last score
  // MFMAs issue the V^T reads of the first two fp8 P.V MFMAs; each P.V MFMA issues those two
  // ahead, and carries two max3 steps of the row max of S(t+1); the reference then moves at
  // every increase (the pages' fp8 recurrence) before the next iteration.
  constexpr bool EXPL8 = D == 256 && C::V8 && MODE != kMaskBlock && KW == 64;
  auto fast_iter_v8 = [&](int t, f32x16* s_cur, f32x16* s_nxt, const unsigned char* kb_nxt,
                          const unsigned char* vb_cur, unsigned char* kb_dma, unsigned char* vb_dma) __attribute__((always_inline)) {
    constexpr int NSM = 2 * C::DK;            // score MFMAs (32)
    constexpr int NPM = C::DTL;               // fp8 P.V MFMAs (8), 64 keys each
    constexpr int NKA = 4;                    // K fragments read ahead
    constexpr int NVA = 2;                    // V^T fragments read ahead
    static_assert(!EXPL8 || (NSM == 32 && NPM == 8), "issue stream shape");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < ntiles) dma_k(key_begin + (t + 2) * BN, kb_dma);
    if (t + 1 < ntiles) dma_v(key_begin + (t + 1) * BN, vb_dma);
    auto kread = [&](int i) __attribute__((always_inline)) {
      const int kt = i / C::DK, kk = i % C::DK;
      return *(const u32x4*)(kb_nxt + k_lane_off + 32 * kt * C::KROWB + (((2 * kk + h) ^ kswz) << 4));
    };
    auto vread = [&](i32x8& a, int dt, int t4) __attribute__((always_inline)) {
      const int row = 16 * t4 + tr8_row;
      const int byte = 32 * dt + tr8_cb;
      const int sw = ((byte >> 4) ^ swz_v<C::VROWB, true>(row)) << 4 | (byte & 15);
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(vb_cur + row * C::VROWB + sw));
      a[2 * t4] = x[0];
      a[2 * t4 + 1] = x[1];
    };
    u32x4 kf[NSM];
    i32x8 vf[NPM];
#pragma unroll
    for (int i = 0; i < NKA; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
    const float neg = -m_ref;
    float psum = 0.f;
    i32x8 pb;
    f32x16 z0, z1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z0[r] = 0.f;
      z1[r] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NSM; ++i) {
      if (i < C::DK) z0 = mfma_qk<C::QK>(kf[i], qf[i % C::DK], z0);
      else z1 = mfma_qk<C::QK>(kf[i], qf[i % C::DK], z1);
      const int j = i + NKA;
      if (j < NSM) kf[j] = kread(j);
      // V^T reads of P.V MFMAs 0 and 1 during the last eight score MFMAs
      if (i >= NSM - 4 * NVA) vread(vf[(i - (NSM - 4 * NVA)) / 4], (i - (NSM - 4 * NVA)) / 4, (i - (NSM - 4 * NVA)) % 4);
      // weight i of P(t): subtile i / 16, register i % 16
      const int kt = i / 16, r = i % 16;
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kt][r], p.c, neg));
      s_cur[kt][r] = e;
      psum += e;
      if ((r & 3) == 3) {
        const int r4 = r - 3;
        int word = __builtin_amdgcn_cvt_pk_bf8_f32(s_cur[kt][r4], s_cur[kt][r4 + 1], 0, false);
        word = __builtin_amdgcn_cvt_pk_bf8_f32(s_cur[kt][r4 + 2], s_cur[kt][r4 + 3], word, true);
        pb[kt * 4 + r4 / 4] = word;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum;
    s_nxt[0] = z0;
    s_nxt[1] = z1;
    __builtin_amdgcn_sched_barrier(0);
    float mk[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int j = 0; j < NPM; ++j) {
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[j], pb, acc[j], 1, 1, 0, 0, 0, 0);
      if (j + NVA < NPM) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) vread(vf[j + NVA], j + NVA, t4);
      }
      // two max3 steps of S(t+1) per P.V MFMA: subtile 0 first, subtile 1 (last score MFMA still
      // running at the start) in the second half
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int step = 2 * j + q, kt = step / 8, r = 2 * (step % 8);
        mk[kt] = max3(mk[kt], s_nxt[kt][r], s_nxt[kt][r + 1]);
        asm("" : "+v"(mk[kt]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float mx = __builtin_fmaxf(mk[0], mk[1]);
    mx = __builtin_fmaxf(mx, partner(mx));
    rescale_to(mx * p.c);
  };

  f32x16 sA[C::KT], sB[C::KT];
  if (ntiles > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bool live0[C::KT], masked0[C::KT];
    tile_flags(0, 0 < nfull, live0, masked0);
    u32x4 fr0[C::KT][C::DK];
    k_frags(fr0, lk0, live0, kswz);
    scores(sA, fr0, lk0, live0, kswz);
    // the explicit unmasked iterations expect the row max of their tile taken beforehand
    if constexpr (EXPL || EXPL8) softmax_max(0, sA, live0, masked0);
  }
  int t = 0;
  // Unmasked iterations (tiles t and t+1 both unmasked) in pairs with fixed buffers.
  for (; t + 2 < nfull; t += 2) {
    if constexpr (EXPL) {
      fast_iter_expl(t, sA, sB, lk1, lv0, lk0, lv1);
      fast_iter_expl(t + 1, sB, sA, lk0, lv1, lk1, lv0);
    } else if constexpr (EXPL8) {
      fast_iter_v8(t, sA, sB, lk1, lv0, lk0, lv1);
      fast_iter_v8(t + 1, sB, sA, lk0, lv1, lk1, lv0);
    } else {
      iteration(true, t, sA, sB, lk1, lv0, lk0, lv1);
      iteration(true, t + 1, sB, sA, lk0, lv1, lk1, lv0);
    }
  }
  // The rest (t is even here), also in pairs with fixed buffers: with buffers chosen at run time
  // the compiler cannot tell the DMA target from the buffer read and waits for the DMA first.
  for (; t < ntiles; t += 2) {
    iteration(false, t, sA, sB, lk1, lv0, lk0, lv1);
    if (t + 1 < ntiles) iteration(false, t + 1, sB, sA, lk0, lv1, lk1, lv0);
  }

  // ---- epilogue: O = acc / l, rounded to Q's type; optional natural-log normaliser -------
  const float l_norm = C::HAT ? l_hat : l_run;
  const float inv = 1.0f / (l_norm + partner(l_norm));
  const float l_exact = LSE ? l_run + partner(l_run) : 0.f;   // (all lanes take part)
  if (my_q < L) {
    unsigned char* orow = p.o + (size_t)(bi * p.lo.sb + hi * p.lo.sh + (long long)my_q * p.lo.sr) * 2;
#pragma unroll
    for (int dt = 0; dt < C::DTL; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        // registers 4*a4 .. 4*a4+3 hold d = 32*dt + 8*a4 + 4*h + 0..3
        if (32 * dt + 8 * a4 >= D) continue;      // padded head dim: nothing to store
        u32x2 w;
        w[0] = pack2<C::QK>(acc[dt][4 * a4] * inv, acc[dt][4 * a4 + 1] * inv);
        w[1] = pack2<C::QK>(acc[dt][4 * a4 + 2] * inv, acc[dt][4 * a4 + 3] * inv);
        *(u32x2*)(orow + (32 * dt + 8 * a4 + 4 * h) * 2) = w;
      }
    if (LSE && h == 0) p.lse[(size_t)bh * L + my_q] = (m_ref + __builtin_amdgcn_logf(l_exact)) * kLn2;
  }
}

// ------------------------------------------------------------------------------------------
// Host side: instance table and launch (argument checks: attn_api.cpp).
// ------------------------------------------------------------------------------------------

template <int D, int DT, int MODE, int NW, int BN, int KW = BN>
hipError_t launch(const Params& p0, hipStream_t stream) {
  using C = Cfg<D, DT, MODE, NW, BN, KW>;
  Params p = p0;
  p.n_qblocks = (p.L + C::BM - 1) / C::BM;
  const long long blocks = (long long)p.n_qblocks * p.bh;
  // causal head groups: the largest divisor of the heads per XCD whose K/V fits the 4 MiB L2
  p.group = 1;
  p.tail = 0;   // (measured: no gain here at head dims 128 and 256)
  if (MODE == kMaskCausal && p.bh % 8 == 0) {
    const long long head_kv = (long long)p.L * D * (2 + C::VB);
    const int hx = p.bh / 8;
    for (int g = hx; g >= 1; --g)
      if (hx % g == 0 && g * head_kv <= (4ll << 20)) {
        p.group = g;
        break;
      }
  }
  if (p.lse != nullptr)
    hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MODE, NW, BN, KW, true>), dim3((unsigned)blocks),
                       dim3(C::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, DT, MODE, NW, BN, KW, false>), dim3((unsigned)blocks),
                       dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

// Launch arguments of a validated call in the kernels' form.
inline Params make_params(const attn::LaunchArgs& a) {
  Params p{};
  p.q = (const unsigned char*)a.q;
  p.k = (const unsigned char*)a.k;
  p.v = (const unsigned char*)a.v;
  p.o = (unsigned char*)a.o;
  p.lse = a.lse;
  p.lq = a.lq;
  p.lk = a.lk;
  p.lv = a.lv;
  p.lo = a.lo;
  p.heads = a.heads;
  p.L = a.L;
  p.bh = a.bh;
  p.c = a.c;
  return p;
}

}  // namespace
