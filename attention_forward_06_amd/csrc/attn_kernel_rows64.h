// Head dims 16, 32 and 64, none and causal, 16-bit V: 64 query rows per wave.
//
// Same online softmax as attn_fwd_kernel ("Triton-CUDA Attention", online-softmax core;
// "Fused Attention", _attn_fwd_inner: running max, running sum, rescaled accumulator, O = acc / l),
// same operand layouts (S^T = K * Q^T with the key permutation pi, O^T = V^T * P^T with
// transposing V reads), same LDS-DMA tile staging.  What differs is the work of one wave: two
// groups of 32 query rows (row group r holds rows qw0 + 32 r + lane % 32), so every K fragment and
// every V^T fragment read from LDS feeds two MFMAs instead of one.  At these head dims one SIMD
// issuing the MFMAs, their LDS operand reads and the softmax VALU work of two waves is what bounds
// the 32-row kernel; halving the LDS reads per MFMA moves that bound.  Registers at head dim 64:
// Q fragments 2 x 16, accumulators 2 x 32, scores 2 x 32, K or V^T fragments 32 -- two waves per
// SIMD still fit; head dim 16 fits three.
//
// Per key tile (64 keys) and wave, the unmasked iteration issues four phases of MFMAs:
//   A  scores of row group 0 (K fragments read once, kept),
//   B  scores of row group 1 from the same K fragments, while the VALU exponentiates row
//      group 0's weights,
//   C  P.V of row group 0 (V^T fragments read once, kept), while the VALU exponentiates row
//      group 1's weights,
//   D  P.V of row group 1 from the same V^T fragments.
// Tiles are not pipelined across iterations (the second row group gives each phase's VALU work
// MFMAs to hide under); K and V of tile t+1 stream into the other LDS buffer during tile t.
// The unmasked iteration takes no row max unless a tile's sum of rounded weights exceeds
// SUM_CAP in some row (a lazy reference, exact in real arithmetic for any reference).  The causal
// diagonal and a ragged tail take the general iteration (mask, row max, capped rescale), one row
// group after the other.  Head dim 16 runs 32-wide tiles whose upper half is zero (as
// attn_fwd_kernel does); its score MFMAs skip that half.
#pragma once

#include "attn_kernel.h"

namespace {

template <int D, int DT, int MODE, bool LSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 16 ? 3 : 2)))
void attn_fwd_rows64_kernel(Params p) {
  constexpr int NW = 4, BN = 64, RG = 2;
  using C = Cfg<D, DT, MODE, NW, BN>;   // tile, DMA and swizzle constants (C::BM is not this kernel's)
  constexpr int BM = 64 * NW;           // query rows per workgroup
  // DK: 16-wide d chunks holding data (head dim 16 runs 32-wide tiles whose upper half is zero;
  // its score MFMAs skip that half)
  constexpr int DK = (D + 15) / 16, DTL = C::DTL;
  static_assert(!C::V8 && MODE != kMaskBlock && C::KT == 2 && D <= 64, "head dim 16-64, 16-bit");
  __shared__ __attribute__((aligned(1024))) unsigned char lk0[C::KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char lv0[C::VTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char lk1[C::KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char lv1[C::VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  int bh, qb;
  block_coords(blockIdx.x, gridDim.x, p.n_qblocks, MODE == kMaskCausal, p.group, p.tail, bh, qb);
  const int L = p.L;
  const int m0 = qb * BM;
  const int qw0 = m0 + 64 * wave;   // the wave's rows: [qw0, qw0 + 64)

  const int bi = bh / p.heads, hi = bh - bi * p.heads;
  const unsigned char* qh = p.q + (size_t)(bi * p.lq.sb + hi * p.lq.sh) * 2;
  const unsigned char* kh = p.k + (size_t)(bi * p.lk.sb + hi * p.lk.sh) * 2;
  const unsigned char* vh = p.v + (size_t)(bi * p.lv.sb + hi * p.lv.sh) * 2;
  const int q_rs = p.lq.sr * 2, k_rs = p.lk.sr * 2, v_rs = p.lv.sr * 2;
  const unsigned q_ext = (unsigned)((L - 1) * q_rs + D * 2);
  const unsigned k_oob = (unsigned)((L - 1) * k_rs + D * 2);
  const unsigned v_oob = (unsigned)((L - 1) * v_rs + D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, q_ext);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, k_oob);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, v_oob);

  // LDS-DMA lane offsets, as in attn_fwd_kernel (the chunks of a padded row, D = 16, point past
  // the buffer and read as zeros).
  constexpr unsigned kPadOff = 0x80000000u;
  unsigned k_off[C::KPER], v_off[C::VPER];
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) {
    const int byte = (wave + i * NW) * 1024 + lane * 16;
    const int row = byte / C::KROWB;
    const int lch = ((byte % C::KROWB) >> 4) ^ swz_k<C::KROWB>(row);
    const int rin = (wave * 1024 + lane * 16) / C::KROWB;
    k_off[i] = lch * 16 < C::KGROWB ? (unsigned)(rin * k_rs + lch * 16) : kPadOff;
  }
#pragma unroll
  for (int i = 0; i < C::VPER; ++i) {
    const int byte = (wave + i * NW) * 1024 + lane * 16;
    const int row = byte / C::VROWB;
    const int lch = ((byte % C::VROWB) >> 4) ^ swz_v<C::VROWB, false>(row);
    const int rin = (wave * 1024 + lane * 16) / C::VROWB;
    v_off[i] = lch * 16 < C::VGROWB ? (unsigned)(rin * v_rs + lch * 16) : kPadOff;
  }
  auto dma_k = [&](int key0, unsigned char* kb) __attribute__((always_inline)) {
    if (key0 + BN <= L) dma_rows<C::KROWB, C::KDMA, C::KPER, NW, BN>(rk, key0, L, k_rs, wave, lane, k_oob, k_off, kb, true);
    else dma_rows<C::KROWB, C::KDMA, C::KPER, NW, BN>(rk, key0, L, k_rs, wave, lane, k_oob, k_off, kb, false);
  };
  auto dma_v = [&](int key0, unsigned char* vb) __attribute__((always_inline)) {
    if (key0 + BN <= L) dma_rows<C::VROWB, C::VDMA, C::VPER, NW, BN>(rv, key0, L, v_rs, wave, lane, v_oob, v_off, vb, true);
    else dma_rows<C::VROWB, C::VDMA, C::VPER, NW, BN>(rv, key0, L, v_rs, wave, lane, v_oob, v_off, vb, false);
  };

  const int key_end = MODE == kMaskCausal ? min(L, m0 + BM) : L;
  const int ntiles = (key_end + BN - 1) / BN;
  // tiles [0, nfull) are visible to every query row of the workgroup
  const int nfull = MODE == kMaskCausal ? min(ntiles, m0 / BN) : min(ntiles, L / BN);

  // Tile t lives in buffer t % 2; the DMA of tile t+1 starts at the top of iteration t.
  if (ntiles > 0) {
    dma_k(0, lk0);
    dma_v(0, lv0);
  }

  // Q^T fragments of both row groups: lane holds Q[row][16 kk + 8 h .. +7].
  u32x4 qf[RG][DK];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      const int q = qw0 + 32 * r + col;
      const bool in = q < L && 16 * kk + 8 * h < D;   // d >= D: the zero half of a padded row
      const unsigned off = in ? (unsigned)(q * q_rs + (16 * kk + 8 * h) * 2) : q_ext;
      qf[r][kk] = buf_load16(rq, off);
    }

  f32x16 acc[RG][DTL];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][dt][i] = 0.f;
  float m_ref[RG], l_run[RG], l_hat[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    m_ref[r] = -INFINITY;   // reference max (scores * c, log2 domain) of row group r
    l_run[r] = 0.f;         // sum of the unrounded weights (kept only for the log-normaliser)
    l_hat[r] = 0.f;         // sum of the rounded 16-bit weights P.V used
  }

  const int krow = key_of_row(col);
  const int kswz = swz_k<C::KROWB>(krow);
  const int k_lane_off = krow * C::KROWB;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr16_row = 8 * (g16 >> 1) + (s16 >> 2);
  const int tr16_cb = 32 * (g16 & 1) + 8 * (s16 & 3);

  auto kread = [&](const unsigned char* kb, int kt, int kk, int ksw) __attribute__((always_inline)) {
    return *(const u32x4*)(kb + k_lane_off + 32 * kt * C::KROWB + (((2 * kk + h) ^ ksw) << 4));
  };
  // V^T fragment of 16-key chunk cc, 32-wide d tile dt: two transposing 8-byte reads.
  auto vread = [&](const unsigned char* vb, int cc, int dt) __attribute__((always_inline)) {
    u32x4 a;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = 16 * cc + 4 * tt + tr16_row;
      const int byte = 64 * dt + tr16_cb;
      const int sw = ((byte >> 4) ^ swz_v<C::VROWB, false>(row)) << 4 | (byte & 15);
      const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vb + row * C::VROWB + sw));
      __builtin_memcpy((char*)&a + 8 * tt, &x, 8);
    }
    return a;
  };
  auto rescale = [&](int r, float alpha) __attribute__((always_inline)) {
    l_run[r] *= alpha;
    l_hat[r] *= alpha;
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][dt][i] *= alpha;
  };

  // General iteration: any mask, exact row max with the capped rescale, one row group after the
  // other (compiler-scheduled; it runs on the causal diagonal and a ragged tail).
  auto general = [&](int t, const unsigned char* kb, const unsigned char* vb, unsigned char* kb_dma,
                     unsigned char* vb_dma) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA of tile t landed
    __syncthreads();                 // everyone's did; nobody still reads tile t-1
    if (t + 1 < ntiles) {
      dma_k((t + 1) * BN, kb_dma);
      dma_v((t + 1) * BN, vb_dma);
    }
    const int key0 = t * BN;
    int ksw = kswz;
    asm volatile("" : "+v"(ksw));    // recompute the read addresses here, not hold them
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int qr0 = qw0 + 32 * r, my_q = qr0 + col;
      bool live[2], masked[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int n0 = key0 + 32 * kt;
        if constexpr (MODE == kMaskCausal) {
          live[kt] = n0 <= qr0 + 31;
          masked[kt] = n0 + 31 > qr0;
        } else {
          live[kt] = n0 < L;
          masked[kt] = n0 + 31 >= L;
        }
      }
      if (!live[0]) continue;   // wave-uniform; subtile 1 is live only if subtile 0 is
      f32x16 s[2];
      float mk[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (!live[kt]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kt][i] = -INFINITY;
          continue;
        }
        f32x16 z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) z = mfma_qk<C::QK>(kread(kb, kt, kk, ksw), qf[r][kk], z);
        s[kt] = z;
        // register i holds key key0 + 32 kt + 16 (i / 8) + 8 h + i % 8
        if (masked[kt]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kt + 16 * (i >> 3) + 8 * h + (i & 7);
            bool ok;
            if constexpr (MODE == kMaskCausal) ok = key <= my_q;
            else ok = key < L;
            if (!ok) s[kt][i] = -INFINITY;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) mk[kt] = max3(mk[kt], s[kt][i], s[kt][i + 1]);
      }
      float mx = __builtin_fmaxf(mk[0], mk[1]);
      mx = __builtin_fmaxf(mx, partner(mx));
      const float m_cand = mx * p.c;
      const bool need = m_cand > m_ref[r] + C::TAU;   // true on a row's first live tile
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? m_cand : m_ref[r];
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref[r] - m_new) : 1.0f;   // 0 at first
        m_ref[r] = m_new;
        rescale(r, alpha);
      }
      const float neg = -m_ref[r];
      u32x4 pk[BN / 16];
      float lh = 0.f, le = 0.f;
#pragma unroll
      for (int cc = 0; cc < BN / 16; ++cc) {
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
      l_hat[r] += lh;
      if constexpr (LSE) l_run[r] += le;
#pragma unroll
      for (int cc = 0; cc < BN / 16; ++cc) {
        if (!live[cc >> 1]) continue;
#pragma unroll
        for (int dt = 0; dt < DTL; ++dt) acc[r][dt] = mfma_qk<DT>(vread(vb, cc, dt), pk[cc], acc[r][dt]);
      }
    }
  };

  // Unmasked iteration: the four phases of the header comment, each MFMA closing a scheduling
  // group with its share of LDS reads and VALU work.  Exponential pair-item k of a row group
  // (chunk k / 4, pair k % 4: two FMAs, two exponentials, one pack, one pair sum) rides on the
  // MFMAs of phase B (row group 0) or C (row group 1), spread evenly, pipelined one deep
  // (exponentials of item k, pack and sum of item k - 1).  A tile sum of at most SUM_CAP = 2^12
  // bounds every weight far inside binary16 and bfloat16.
  constexpr float SUM_CAP = 4096.f;
  auto fast = [&](int t, const unsigned char* kb, const unsigned char* vb, unsigned char* kb_dma,
                  unsigned char* vb_dma) __attribute__((always_inline)) {
    constexpr int NS = 2 * DK;            // score MFMAs per row group (8)
    constexpr int NP = (BN / 16) * DTL;   // P.V MFMAs per row group (8)
    constexpr int NKA = NS < 4 ? NS : 4;  // K fragments read ahead
    constexpr int NVA = NS < 4 ? NS : 4;  // V^T fragments read ahead
    constexpr int NIT = (BN / 16) * 4;    // pair-items per row group (16)
    constexpr int IPB = NIT / NS;         // pair-items per score MFMA of phase B
    constexpr int IPC = NIT / NP;         // pair-items per P.V MFMA of phase C
    static_assert(NIT == IPB * NS && NIT == IPC * NP && NVA <= NS, "issue stream shape");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) {
      dma_k((t + 1) * BN, kb_dma);
      dma_v((t + 1) * BN, vb_dma);
    }
    u32x4 kf[NS], vf[NP];
#pragma unroll
    for (int i = 0; i < NKA; ++i) kf[i] = kread(kb, i / DK, i % DK, kswz);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 z[RG][2];
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        z[r][0][i] = 0.f;
        z[r][1][i] = 0.f;
      }
    u32x4 pk[RG][BN / 16];
    float lh[RG] = {0.f, 0.f}, le[RG] = {0.f, 0.f};
    float e0[NIT], e1[NIT];
    auto item_exp = [&](int r, int k, float neg) __attribute__((always_inline)) {
      const int cc = k >> 2, w = k & 3, kt = cc >> 1, c8 = (cc & 1) * 8;
      e0[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[r][kt][c8 + 2 * w], p.c, neg));
      e1[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[r][kt][c8 + 2 * w + 1], p.c, neg));
    };
    auto item_pack = [&](int r, int k) __attribute__((always_inline)) {
      const int cc = k >> 2, w = k & 3;
      pk[r][cc][w] = pack2<DT>(e0[k], e1[k]);
      lh[r] = sum2_acc<DT>(pk[r][cc][w], lh[r]);
      if constexpr (LSE) le[r] += e0[k] + e1[k];
    };
    // rare: some row's tile sum exceeds the cap, so one weight may have -- exact row max, the
    // reference moved at any increase, the weights again
    auto lazy_check = [&](int r) __attribute__((always_inline)) {
      if (__builtin_amdgcn_ballot_w64(lh[r] > SUM_CAP)) {
        float mk[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; i += 2) mk[kt] = max3(mk[kt], z[r][kt][i], z[r][kt][i + 1]);
        float mx = __builtin_fmaxf(mk[0], mk[1]);
        mx = __builtin_fmaxf(mx, partner(mx)) * p.c;
        const bool up = mx > m_ref[r];
        if (__builtin_amdgcn_ballot_w64(up)) {
          const float alpha = up ? __builtin_amdgcn_exp2f(m_ref[r] - mx) : 1.0f;
          m_ref[r] = up ? mx : m_ref[r];
          rescale(r, alpha);
        }
        lh[r] = 0.f;
        le[r] = 0.f;
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
          item_exp(r, k, -m_ref[r]);
          item_pack(r, k);
        }
      }
      l_hat[r] += lh[r];
      if constexpr (LSE) l_run[r] += le[r];
    };

    // A: scores of row group 0
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      z[0][i / DK] = mfma_qk<C::QK>(kf[i], qf[0][i % DK], z[0][i / DK]);
      if (i + NKA < NS) kf[i + NKA] = kread(kb, (i + NKA) / DK, (i + NKA) % DK, kswz);
      __builtin_amdgcn_sched_barrier(0);
    }
    // B: scores of row group 1 from the same K fragments; weights of row group 0; the first
    // V^T reads during the last MFMAs
    const float neg0 = -m_ref[0];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      z[1][i / DK] = mfma_qk<C::QK>(kf[i], qf[1][i % DK], z[1][i / DK]);
      if (i >= NS - NVA) {
        const int j = i - (NS - NVA);
        vf[j] = vread(vb, j / DTL, j % DTL);
      }
#pragma unroll
      for (int q = 0; q < IPB; ++q) {
        const int k = i * IPB + q;
        item_exp(0, k, neg0);
        if (k > 0) item_pack(0, k - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    item_pack(0, NIT - 1);
    lazy_check(0);
    __builtin_amdgcn_sched_barrier(0);
    // C: P.V of row group 0 (V^T fragments kept); weights of row group 1
    const float neg1 = -m_ref[1];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      acc[0][j % DTL] = mfma_qk<DT>(vf[j], pk[0][j / DTL], acc[0][j % DTL]);
      if (j + NVA < NP) vf[j + NVA] = vread(vb, (j + NVA) / DTL, (j + NVA) % DTL);
#pragma unroll
      for (int q = 0; q < IPC; ++q) {
        const int k = j * IPC + q;
        item_exp(1, k, neg1);
        if (k > 0) item_pack(1, k - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    item_pack(1, NIT - 1);
    lazy_check(1);
    __builtin_amdgcn_sched_barrier(0);
    // D: P.V of row group 1 from the same V^T fragments
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      acc[1][j % DTL] = mfma_qk<DT>(vf[j], pk[1][j / DTL], acc[1][j % DTL]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The unmasked tiles first, in pairs with fixed buffers (tile t in buffer t % 2: with buffers
  // chosen at run time the compiler cannot tell the DMA target from the buffer read and waits
  // for the DMA first), then the rest.  Tile 0 may take the unmasked iteration: its reference
  // is still -inf, so every weight is +inf, the cap check fires and the recomputation sets the
  // reference to the tile's exact row max (the accumulator, all zeros, is scaled by 0).
  int t = 0;
  for (; t + 1 < nfull; t += 2) {
    fast(t, lk0, lv0, lk1, lv1);
    fast(t + 1, lk1, lv1, lk0, lv0);
  }
  if (t < nfull) {   // t is even here
    fast(t, lk0, lv0, lk1, lv1);
    ++t;
  }
  for (; t < ntiles; ++t) {
    if (t & 1) general(t, lk1, lv1, lk0, lv0);
    else general(t, lk0, lv0, lk1, lv1);
  }

  // ---- epilogue: O = acc / l, rounded to Q's type; optional natural-log normaliser ----------
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const float inv = 1.0f / (l_hat[r] + partner(l_hat[r]));
    const float l_exact = LSE ? l_run[r] + partner(l_run[r]) : 0.f;   // (all lanes take part)
    const int my_q = qw0 + 32 * r + col;
    if (my_q < L) {
      unsigned char* orow = p.o + (size_t)(bi * p.lo.sb + hi * p.lo.sh + (long long)my_q * p.lo.sr) * 2;
#pragma unroll
      for (int dt = 0; dt < DTL; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          // registers 4 a4 .. 4 a4 + 3 hold d = 32 dt + 8 a4 + 4 h + 0..3
          if (32 * dt + 8 * a4 >= D) continue;      // padded head dim: nothing to store
          u32x2 w;
          w[0] = pack2<C::QK>(acc[r][dt][4 * a4] * inv, acc[r][dt][4 * a4 + 1] * inv);
          w[1] = pack2<C::QK>(acc[r][dt][4 * a4 + 2] * inv, acc[r][dt][4 * a4 + 3] * inv);
          *(u32x2*)(orow + (32 * dt + 8 * a4 + 4 * h) * 2) = w;
        }
      if (LSE && h == 0) p.lse[(size_t)bh * L + my_q] = (m_ref[r] + __builtin_amdgcn_logf(l_exact)) * kLn2;
    }
  }
}

// Launch of the 64-rows-per-wave kernel: 256 query rows per workgroup.
template <int D, int DT, int MODE>
hipError_t launch_rows64(const Params& p0, hipStream_t stream) {
  constexpr int BM = 256;
  Params p = p0;
  p.n_qblocks = (p.L + BM - 1) / BM;
  const long long blocks = (long long)p.n_qblocks * p.bh;
  // causal head groups: the largest divisor of the heads per XCD whose K/V fits the 4 MiB L2;
  // the shortest quarter of every head's query blocks runs after all the others (block_coords)
  p.group = 1;
  p.tail = p.n_qblocks / 4;
  if (MODE == kMaskCausal && p.bh % 8 == 0) {
    const long long head_kv = (long long)p.L * D * 4;
    const int hx = p.bh / 8;
    for (int g = hx; g >= 1; --g)
      if (hx % g == 0 && g * head_kv <= (4ll << 20)) {
        p.group = g;
        break;
      }
  }
  if (p.lse != nullptr)
    hipLaunchKernelGGL((attn_fwd_rows64_kernel<D, DT, MODE, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_rows64_kernel<D, DT, MODE, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace
