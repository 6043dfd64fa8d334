// attn_fwd_kernels.h -- the attention-forward kernels of libattn.so: the
// "simple", "pipelined" and "pingpong" schedules, all built from the
// per-block step helpers of attn_common.h (same arithmetic, bit for bit).
// Included by attn_fwd.hip, which instantiates them for its variant table.
#ifndef ATTN_FWD_KERNELS_H
#define ATTN_FWD_KERNELS_H

#include "attn_common.h"

namespace {

// ---------------------------------------------------------------- simple kernel
// Blocks stream through an ST-slot ring (block j in slot j mod ST): at the
// top of block j every wave waits for its share of block j's copies, meets
// the others at the barrier (so slot (j-1) mod ST is no longer read), and
// starts the copies of block j+ST-1 into that slot; then the steps of block j
// run in program order. The reference schedule the overlapped kernels are
// checked against (bit for bit).
template <int D, int NW, int BN, int QT, bool CAUSAL, int ST, int SLOT>
__device__ __forceinline__ void simple_block(const Ctx& c, char* smem, int j,
                                             const LdsOffsets<D>& off,
                                             const bf16x8 (&qf)[QT][D / 16],
                                             f32x16 (&o)[QT][D / 32], float (&m_run)[QT], float (&ms_run)[QT],
                                             float (&l_run)[QT]) {
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  constexpr int PER_BLOCK = 2 * LD;  // copy instructions per block per wave
  // every block issues its copies (past the last block a clamped duplicate
  // lands in a free slot), so the count of younger copies is always exact
  wait_vmcnt<(ST - 2) * PER_BLOCK>();  // blocks j+1 .. j+ST-2 may stay in flight
  block_barrier();
  constexpr int NS = (SLOT + ST - 1) % ST;
  const int row_next = min(j + ST - 1, c.nblk - 1) * BN;
  const int kv0 = j * BN;
  if (kv0 >= c.kv_end_w) {  // wave-uniform: the whole block is masked for this wave
#pragma unroll
    for (int t = 0; t < LD; ++t) {
      issue_copy<D, NW, BN, false>(c.Kh, row_next, c.N, k_slot<D, BN, ST>(smem, NS), c.wave, c.lane, t);
      issue_copy<D, NW, BN, true>(c.Vh, row_next, c.N, v_slot<D, BN, ST>(smem, NS), c.wave, c.lane, t);
    }
    return;
  }
  // copies of block j+ST-1 interleaved with the mma_qk stream of block j
  f32x16 s[QT][BN / 32];
  qk_block_with_copies<D, BN, QT, PER_BLOCK>(k_slot<D, BN, ST>(smem, SLOT), off, qf, s, [&](int ci) {
    const int t = ci >> 1;
    if (ci & 1)
      issue_copy<D, NW, BN, true>(c.Vh, row_next, c.N, v_slot<D, BN, ST>(smem, NS), c.wave, c.lane, t);
    else
      issue_copy<D, NW, BN, false>(c.Kh, row_next, c.N, k_slot<D, BN, ST>(smem, NS), c.wave, c.lane, t);
  });
  sched_mfma_with_reads<(D / 16) * (BN / 32), 1, QT, kPfQK>();
  if (block_needs_mask<BN, CAUSAL>(c, kv0)) mask_block<BN, QT, CAUSAL>(s, kv0, c.qi0, c.N, c.lane);
  bf16x8 pb[QT][BN / 16];
  float alpha[QT];
  softmax_block<BN, QT>(s, pb, c.c_log2, m_run, ms_run, l_run, alpha);
  rescale_block<D, QT>(o, alpha);
  pv_block<D, BN, QT>(v_slot<D, BN, ST>(smem, SLOT), off, pb, o);
  sched_mfma_with_reads<(BN / 16) * (D / 32), 2, QT, kPfPV>();
}

// OCC = workgroups per CU the register budget is sized for (waves per SIMD =
// NW * OCC / 4): with NW = 4 and OCC = 2 two independent workgroups share a
// CU, so the two waves on each SIMD are never held in step by one barrier.
template <int D, int NW, int BN, int QT, bool CAUSAL, int ST, int OCC>
__device__ __forceinline__ void attn_fwd_simple_tile(const Ctx& c, char* smem,
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, ST>;

  // Q first, then blocks 0 .. ST-2 (so the in-loop waits count block copies
  // only); past the last block a clamped duplicate lands in a slot nobody
  // reads, so that every block's wait counts exactly ST-2 younger blocks
  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, q_mode, qf, c.lane);
  if constexpr (NW * OCC <= 4) park_in_agprs<QT, D / 16>(qf);
#pragma unroll
  for (int b = 0; b < ST - 1; ++b) {
    const int row = min(b, c.nblk - 1) * BN;
    issue_block_load<D, NW, BN, false>(c.Kh, row, N, k_slot<D, BN, ST>(smem, b), c.wave, c.lane);
    issue_block_load<D, NW, BN, true>(c.Vh, row, N, v_slot<D, BN, ST>(smem, b), c.wave, c.lane);
  }
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], ms_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
    ms_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }
  for (int j = 0; j < c.nblk; j += ST) {
    simple_block<D, NW, BN, QT, CAUSAL, ST, 0>(c, smem, j, off, qf, o, m_run, ms_run, l_run);
    if (j + 1 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 1 % ST>(c, smem, j + 1, off, qf, o, m_run, ms_run, l_run);
    if (ST > 2 && j + 2 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 2 % ST>(c, smem, j + 2, off, qf, o, m_run, ms_run, l_run);
    if (ST > 3 && j + 3 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 3 % ST>(c, smem, j + 3, off, qf, o, m_run, ms_run, l_run);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, ms_run, l_run, c.c_log2, c.lane);
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int ST, int OCC>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_simple(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, ST>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  if constexpr (!CAUSAL) {
    Ctx c;
    make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, 0, c);
    attn_fwd_simple_tile<D, NW, BN, QT, CAUSAL, ST, OCC>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
  } else {
    for (int pass = 0; pass < 2; ++pass) {
      Ctx c;
      if (!make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, pass, c)) break;
      if (pass > 0) block_barrier();  // every wave is done with the ring of the previous tile
      attn_fwd_simple_tile<D, NW, BN, QT, CAUSAL, ST, OCC>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
    }
  }
}

// ---------------------------------------------------------------- pipelined kernel
// Software-pipelined schedule inside each wave (the pages' FlashAttention-
// forward schedule found by Twill, section 3.1 of the software-pipelining
// page: the first GEMM is hoisted into the loop prologue so exp latency is
// never exposed, and one tile's softmax overlaps the other GEMMs), restated
// for gfx950. A wave's MFMAs run alongside its own VALU work, so every phase
// gives the wave both kinds of work:
//   prologue : K_0 .. K_{ST-1}, V_0 .. V_{ST-3} -> LDS; S_0 = Q K_0^T
//   block j  : (a) mma_pv(V_{j-1}, P_{j-1})  with  mask, row max and the
//                  first half of the exp units of S_j;
//              (b) mma_qk(K_{j+1}) -> S_{j+1}  with  the other exp units,
//                  row sums and packing of P_j;
//              then O *= alpha_j per query tile (skipped for a tile when no
//              row of it moved its max)
//   epilogue : mma_pv(V_{n-1}, P_{n-1})
// An exp unit is one (query tile, 32-key tile) pair, taken query-tile-major,
// so with one key tile and two query tiles each phase gets one tile's exps.
// O sees exactly the simple schedule's sequence of updates (... += P_{j-1}V,
// *= alpha_j, += P_j V ...), so results agree bit for bit. LDS holds ST K
// and ST V slots (K_i and V_i in slot i mod ST). At the top of block j each
// wave waits for its copies of K_{j+1} and V_{j-1} (those of the last ST-2
// blocks may stay in flight), meets the others at the barrier (after which
// K_j and V_{j-2} are no longer read) and, spread through phase (b), copies
// K_{j+ST} over K_j and V_{j+ST-2} over V_{j-2}: ST-1 blocks of latency.

// MFMA stream of NR read groups (RD reads each, feeding MR MFMAs) with NV
// VALU instructions after every MFMA and NVM VMEM copies spread over the
// steady part; reads run PF groups ahead.
template <int I, int NR, int PF, int RD, int MR, int NV, int NVM>
__device__ __forceinline__ void sched_valu_steps() {
  if constexpr (I < NR - PF) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    constexpr int due = copies_due<NR, PF, NVM>(I);
    if constexpr (due > 0) __builtin_amdgcn_sched_group_barrier(0x010, due, 0);
    sched_valu_steps<I + 1, NR, PF, RD, MR, NV, NVM>();
  }
}
template <int NR, int RD, int MR, int PF, int NV, int NVM>
__device__ __forceinline__ void sched_mfma_reads_valu_copies() {
  __builtin_amdgcn_sched_group_barrier(0x100, RD * PF, 0);
  sched_valu_steps<0, NR, PF, RD, MR, NV, NVM>();
#pragma unroll
  for (int i = 0; i < PF * MR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

template <int D, int NW, int BN, int ST, int SLOT>
__device__ __forceinline__ auto pipe_top(const Ctx& c, char* smem, int j) {
  constexpr int PER_BLOCK = 2 * Tile<D, NW, BN>::LOADS;  // copies per block per wave
  wait_vmcnt<(ST - 2) * PER_BLOCK>();
  block_barrier();
  // past the last block a clamped duplicate lands in a slot nobody reads again
  const int row_k = min(j + ST, c.nblk - 1) * BN;
  const int row_v = min(j + ST - 2, c.nblk - 1) * BN;
  return [&c, smem, row_k, row_v](int ci) {
    const int t = ci >> 1;
    if (ci & 1)
      issue_copy<D, NW, BN, true>(c.Vh, row_v, c.N, v_slot<D, BN, ST>(smem, (SLOT + ST - 2) % ST), c.wave,
                                  c.lane, t);
    else
      issue_copy<D, NW, BN, false>(c.Kh, row_k, c.N, k_slot<D, BN, ST>(smem, SLOT), c.wave, c.lane, t);
  };
}

// Exp units [U0, U1) of S (unit u = query tile u / NB, key tile u % NB).
template <int BN, int QT, int U0, int U1>
__device__ __forceinline__ void softmax_exp_units(f32x16 (&s)[QT][BN / 32], float c_log2,
                                                  const float (&m_run)[QT], float (&ps)[QT][4]) {
  constexpr int NB = BN / 32;
  static_for_from<U0, U1>([&](auto U) {
    constexpr int qt = U / NB, kb = U % NB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][kb][r], c_log2, -m_run[qt]));
      s[qt][kb][r] = p;
      if (kb == 0 && r < 4) ps[qt][r] = p;
      else ps[qt][r & 3] += p;
    }
  });
}

// Block j when the whole workgroup has P_{j-1}, an unmasked S_j and a next
// block: both phases overlapped.
template <int D, int NW, int BN, int QT, int ST, int SLOT>
__device__ __forceinline__ void pipe_block_fast(const Ctx& c, char* smem, int j, const LdsOffsets<D>& off,
                                                const bf16x8 (&qf)[QT][D / 16],
                                                f32x16 (&s_cur)[QT][BN / 32],
                                                f32x16 (&s_nxt)[QT][BN / 32], bf16x8 (&pb)[QT][BN / 16],
                                                f32x16 (&o)[QT][D / 32], float (&m_run)[QT], float (&ms_run)[QT],
                                                float (&l_run)[QT]) {
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  constexpr int NB = BN / 32;
  constexpr int NU = QT * NB, UA = (NU + 1) / 2;  // exp units, and those of phase (a)
  constexpr int MA = (BN / 16) * (D / 32) * QT, MB = (D / 16) * NB * QT;  // MFMAs per phase
  // VALU instructions placed after each MFMA: with one query tile the tuned
  // 5 and 4; else about the phase's count (an exp unit is 16 fma, exp and
  // add; stats take 8 max3 per key tile plus 6; packing and the sums 8 per
  // key tile plus 4 per query tile) over its MFMAs
  constexpr int NVA = QT == 1 ? 5 : (QT * (8 * NB + 6) + UA * 48 + MA - 1) / MA;
  constexpr int NVB = QT == 1 ? 4 : ((NU - UA) * 48 + QT * (8 * NB + 4) + MB - 1) / MB;
  auto copy = pipe_top<D, NW, BN, ST, SLOT>(c, smem, j);
  float alpha[QT], ps[QT][4];
  // (a) mma_pv(V_{j-1}) with the row maxima and the first exp units
  pv_block<D, BN, QT>(v_slot<D, BN, ST>(smem, (SLOT + ST - 1) % ST), off, pb, o);
  softmax_stats<BN, QT>(s_cur, c.c_log2, m_run, ms_run, alpha);
  softmax_exp_units<BN, QT, 0, UA>(s_cur, c.c_log2, m_run, ps);
  static_for<UA>([&](auto U) {
    pin(s_cur[U / NB][U % NB]);
    if constexpr (U % NB == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pin(ps[U / NB][e]);
    }
  });
  sched_mfma_reads_valu_copies<(BN / 16) * (D / 32), 2, QT, kPfPV, NVA, 0>();
  __builtin_amdgcn_sched_barrier(0);
  // (b) mma_qk(K_{j+1}) with this block's copies, the remaining exp units, row
  // sums and packing. (Copies sit among the K reads: plain LDS loads whose
  // addresses the compiler can tell apart from the copy destinations; next to
  // the transposing V reads it would wait for every copy to land.)
  qk_block_with_copies<D, BN, QT, 2 * LD>(k_slot<D, BN, ST>(smem, (SLOT + 1) % ST), off, qf, s_nxt, copy);
  softmax_exp_units<BN, QT, UA, NU>(s_cur, c.c_log2, m_run, ps);
  softmax_sum<QT>(l_run, alpha, ps);
  softmax_pack<BN, QT>(s_cur, pb);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    pin(l_run[qt]);
#pragma unroll
    for (int p = 0; p < BN / 16; ++p) pin(pb[qt][p]);
  }
  sched_mfma_reads_valu_copies<(D / 16) * NB, 1, QT, kPfQK, NVB, 2 * LD>();
  __builtin_amdgcn_sched_barrier(0);
  rescale_block<D, QT>(o, alpha);
}

// Any block (first, masked, past a wave's causal limit, last): the same
// steps in the same order, without overlap.
template <int D, int NW, int BN, int QT, bool CAUSAL, int ST, int SLOT>
__device__ __forceinline__ void pipe_block_generic(const Ctx& c, char* smem, int j,
                                                   const LdsOffsets<D>& off,
                                                   const bf16x8 (&qf)[QT][D / 16],
                                                   f32x16 (&s_cur)[QT][BN / 32],
                                                   f32x16 (&s_nxt)[QT][BN / 32],
                                                   bf16x8 (&pb)[QT][BN / 16], f32x16 (&o)[QT][D / 32],
                                                   float (&m_run)[QT], float (&ms_run)[QT], float (&l_run)[QT]) {
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  constexpr int NB = BN / 32;
  auto copy = pipe_top<D, NW, BN, ST, SLOT>(c, smem, j);
#pragma unroll
  for (int ci = 0; ci < 2 * LD; ++ci) copy(ci);
  const int kv0 = j * BN;
  const bool act = kv0 < c.kv_end_w;                         // S_j has live keys (wave-uniform)
  const bool prv = j > 0 && kv0 - BN < c.kv_end_w;           // P_{j-1} exists
  const bool nxt = j + 1 < c.nblk && kv0 + BN < c.kv_end_w;  // S_{j+1} is needed
  float alpha[QT], ps[QT][4];
  if (prv) {
    pv_block<D, BN, QT>(v_slot<D, BN, ST>(smem, (SLOT + ST - 1) % ST), off, pb, o);
    sched_mfma_with_reads<(BN / 16) * (D / 32), 2, QT, kPfPV>();
  }
  if (act) {
    if (block_needs_mask<BN, CAUSAL>(c, kv0)) mask_block<BN, QT, CAUSAL>(s_cur, kv0, c.qi0, c.N, c.lane);
    softmax_stats<BN, QT>(s_cur, c.c_log2, m_run, ms_run, alpha);
    softmax_exp_units<BN, QT, 0, (QT * NB + 1) / 2>(s_cur, c.c_log2, m_run, ps);
  }
  if (nxt) {
    qk_block<D, BN, QT>(k_slot<D, BN, ST>(smem, (SLOT + 1) % ST), off, qf, s_nxt);
    sched_mfma_with_reads<(D / 16) * NB, 1, QT, kPfQK>();
  }
  if (act) {
    softmax_exp_units<BN, QT, (QT * NB + 1) / 2, QT * NB>(s_cur, c.c_log2, m_run, ps);
    softmax_sum<QT>(l_run, alpha, ps);
    softmax_pack<BN, QT>(s_cur, pb);
    rescale_block<D, QT>(o, alpha);
  }
}

// NW waves, QT query tiles of 32 per wave, BN keys per block, ST ring slots
// (even: the S buffers swap roles every block).
template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int ST>
__device__ __forceinline__ void attn_fwd_pipelined_tile(const Ctx& c, char* smem,
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  static_assert(ST % 2 == 0, "the block loop is unrolled by ST and S alternates by parity");
  using T = Tile<D, NW, BN, QT, ST>;

  // prologue: Q; K_0 .. K_{ST-1} and V_0 .. V_{ST-3} in flight; S_0 = Q K_0^T
  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, q_mode, qf, c.lane);
  if constexpr (NW * OCC <= 4) park_in_agprs<QT, D / 16>(qf);
  static_for<ST>([&](auto I) {
    if (I < c.nblk) {
      issue_block_load<D, NW, BN, false>(c.Kh, I * BN, N, k_slot<D, BN, ST>(smem, I), c.wave, c.lane);
      if constexpr (I + 2 < ST)
        issue_block_load<D, NW, BN, true>(c.Vh, I * BN, N, v_slot<D, BN, ST>(smem, I), c.wave, c.lane);
    }
  });
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], ms_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
    ms_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }
  f32x16 sa[QT][BN / 32], sb[QT][BN / 32];
  bf16x8 pb[QT][BN / 16];
  wait_vmcnt<0>();
  block_barrier();
  qk_block<D, BN, QT>(k_slot<D, BN, ST>(smem, 0), off, qf, sa);  // block 0 is never skipped
  sched_mfma_with_reads<(D / 16) * (BN / 32), 1, QT, kPfQK>();

  // Blocks 1 .. jf-1 take the overlapped path for every wave: they have a
  // previous and a next block, no key past N and (causal) no key past the
  // workgroup's first query. Block 0 and blocks jf .. n-1 take the generic
  // path. Block j uses slot j mod ST; S roles alternate with its parity.
  const int n = c.nblk;
  int jf = n - 1;
  if (N % BN) jf = min(jf, N / BN);
  if (CAUSAL) jf = min(jf, (c.q0 + 1) / BN);
  pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, 0>(c, smem, 0, off, qf, sa, sb, pb, o, m_run, ms_run, l_run);
  int j = 1;
  for (; j + ST - 1 < jf; j += ST) {
    static_for<ST>([&](auto I) {
      constexpr int slot = (1 + I) % ST;
      if constexpr ((1 + I) % 2)
        pipe_block_fast<D, NW, BN, QT, ST, slot>(c, smem, j + I, off, qf, sb, sa, pb, o, m_run, ms_run, l_run);
      else
        pipe_block_fast<D, NW, BN, QT, ST, slot>(c, smem, j + I, off, qf, sa, sb, pb, o, m_run, ms_run, l_run);
    });
  }
  for (; j < n; j += ST) {
    static_for<ST>([&](auto I) {
      constexpr int slot = (1 + I) % ST;
      if (j + I < n) {
        if constexpr ((1 + I) % 2)
          pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, slot>(c, smem, j + I, off, qf, sb, sa, pb, o, m_run, ms_run, l_run);
        else
          pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, slot>(c, smem, j + I, off, qf, sa, sb, pb, o, m_run, ms_run, l_run);
      }
    });
  }
  // epilogue: mma_pv of the last block (V_{n-1} in slot (n-1) mod ST)
  wait_vmcnt<0>();
  block_barrier();
  if ((n - 1) * BN < c.kv_end_w) {
    static_for<ST>([&](auto I) {
      if ((n - 1) % ST == I) pv_block<D, BN, QT>(v_slot<D, BN, ST>(smem, I), off, pb, o);
    });
  }
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, ms_run, l_run, c.c_log2, c.lane);
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int ST>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_pipelined(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, ST>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  if constexpr (!CAUSAL) {
    Ctx c;
    make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, 0, c);
    attn_fwd_pipelined_tile<D, NW, BN, QT, CAUSAL, OCC, ST>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
  } else {
    for (int pass = 0; pass < 2; ++pass) {
      Ctx c;
      if (!make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, pass, c)) break;
      if (pass > 0) block_barrier();  // every wave is done with the ring of the previous tile
      attn_fwd_pipelined_tile<D, NW, BN, QT, CAUSAL, OCC, ST>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
    }
  }
}

// issue_copy through inline assembly (cs_dma): the compiler does not see the
// LDS write, so it adds no wait for it before later LDS reads; callers wait
// explicitly (wait_vmcnt) before anything reads the destination.
template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ void issue_copy_asm(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                               int wave, int lane, int t) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc<D, BN>(src, row0, N);
  const int off = (int)block_lane_offset<D, NW, BN, IS_V>(t, wave, lane);
  cs_dma(r, off, dst + (t * NW + wave) * 64 * 16);
}

// ---------------------------------------------------------------- fused matrix turn
// The ping-pong matrix turn as one instruction stream: mma_pv(V_j) and then
// mma_qk(K_{j+1}) share one scheduling region (no branch or scalar set-up
// between them), so the fragment reads run PF MFMAs ahead of their consumers
// across the boundary between the two products, and the first QK^T MFMAs do
// not wait for LDS. Copies of later blocks are spread over the QK^T part. The
// first NPRE V fragment pairs may already be in registers (read before the
// barrier that opens the turn). Same MFMAs in the same order per
// accumulator as pv_block followed by qk_block, so results are bit-identical.

// V^T fragment pair of P.V read group G (p = G / (D/32), dim tile t = G % (D/32)).
template <int D, int G>
__device__ __forceinline__ void read_v_pair(const char* Vs, const LdsOffsets<D>& off, i16x4 (&va)[2]) {
  constexpr int p = G / (D / 32), t = G % (D / 32);
  va[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Vs + off.v[t] + (p * 16) * (D * 2)));
  va[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Vs + off.v[t] + (p * 16 + 8) * (D * 2)));
}

template <int D, int BN, int NPRE>
struct FusedTurn {
  static constexpr int NT = D / 32, NP = BN / 16;     // P.V: dim tiles, 16-key groups
  static constexpr int NKK = D / 16, NKB = BN / 32;   // QK^T: 16-wide d chunks, 32-key tiles
  static constexpr int NG_PV = NP * NT, NG_QK = NKK * NKB, NG = NG_PV + NG_QK;
  static constexpr int PF = 4;                        // read groups in flight ahead of the MFMAs
  // LDS read instructions of read group g (pre-read groups have none)
  static constexpr int reads(int g) { return g < NPRE ? 0 : (g < NG_PV ? 2 : 1); }
  // copy c of NC is issued right after the reads of group copy_group(c)
  template <int NC>
  static constexpr int copy_group(int c) { return NC > 0 ? NG_PV + PF + (c * (NG_QK - PF)) / NC : NG; }
  template <int NC>
  static constexpr int copies_at(int g) {
    int n = 0;
    for (int c = 0; c < NC; ++c) n += copy_group<NC>(c) == g;
    return n;
  }
};

template <int D, int BN, int QT, int NPRE, int NC, int I>
__device__ __forceinline__ void fused_sched_steps() {
  using F = FusedTurn<D, BN, NPRE>;
  if constexpr (I < F::NG) {
    __builtin_amdgcn_sched_group_barrier(0x008, QT, 0);
    if constexpr (I + F::PF < F::NG) {
      constexpr int r = F::reads(I + F::PF);
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      constexpr int nc = F::template copies_at<NC>(I + F::PF);
      if constexpr (nc > 0) __builtin_amdgcn_sched_group_barrier(0x020, nc, 0);
    }
    fused_sched_steps<D, BN, QT, NPRE, NC, I + 1>();
  }
}

template <int D, int BN, int QT, int NPRE, int NC, int NPA, typename CopyFn>
__device__ __forceinline__ void fused_pv_qk(const char* Vs, const char* Ks, const LdsOffsets<D>& off,
                                            const bf16x8 (&qf)[QT][D / 16], f32x16 (&s)[QT][BN / 32],
                                            const bf16x8 (&pb)[QT][BN / 16], f32x16 (&o)[QT][D / 32],
                                            const i16x4 (&pre)[NPA][2], CopyFn&& copy) {
  using F = FusedTurn<D, BN, NPRE>;
  static_assert(NPA >= NPRE, "pre-read registers");
  static_assert(F::NG_QK > F::PF, "the copies sit in the QK^T part");
  i16x4 va[F::NG_PV][2];
  bf16x8 kf[F::NG_QK];
  // program order: every read, copies among the K reads at their groups
  static_for<F::NG>([&](auto G) {
    constexpr int g = G;
    if constexpr (g < F::NG_PV) {
      if constexpr (g < NPRE) {
        va[g][0] = pre[g][0];
        va[g][1] = pre[g][1];
      } else {
        read_v_pair<D, g>(Vs, off, va[g]);
      }
    } else {
      constexpr int i = g - F::NG_PV, kk = i / F::NKB, kb = i % F::NKB;
      kf[i] = *(LDS_AS const bf16x8*)(Ks + off.k[kk] + kb * 32 * (D * 2));
    }
    static_for<NC>([&](auto C) {
      if constexpr (F::template copy_group<NC>(C) == g) copy(int(C));
    });
  });
  static_for<F::NG_PV>([&](auto G) {
    constexpr int g = G, t = g % F::NT, p = g / F::NT;
    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[g][0], va[g][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[qt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qt][p], o[qt][t], 0, 0, 0);
  });
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < F::NKB; ++kb) s[qt][kb] = f32x16{};
  static_for<F::NG_QK>([&](auto I) {
    constexpr int i = I, kk = i / F::NKB, kb = i % F::NKB;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      s[qt][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[qt][kk], s[qt][kb], 0, 0, 0);
  });
  // schedule: the first PF groups' reads, then per MFMA group the reads (and
  // copies) of the group PF ahead
  constexpr int first = [] {
    int n = 0;
    for (int g = 0; g < F::PF; ++g) n += F::reads(g);
    return n;
  }();
  if constexpr (first > 0) __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
  fused_sched_steps<D, BN, QT, NPRE, NC, 0>();
}

// ---------------------------------------------------------------- ping-pong kernel
// Two wave groups per workgroup (A = waves 0..NW/2-1, B = the rest; each
// SIMD holds one wave of each) alternate on the matrix core, half a block
// apart -- the pages' forward schedule in which two compute groups take turns
// on the matrix unit while the other runs the softmax (software-pipelining
// page, section 3.1), restated for gfx950 with s_barrier as the turn signal.
// Intervals t = 0, 1, ..., 2n (n = KV blocks) are separated by barriers:
//
//   interval   group A                   group B
//   prologue   S_0 = Q K_0^T              -
//   2j         softmax_j (+rescale)       mma_pv(V_{j-1}), S_j = Q K_j^T
//   2j+1       mma_pv(V_j), S_{j+1}       softmax_j (+rescale)
//
// K_j is read in intervals 2j-1 (A) and 2j (B), V_j in 2j+1 (A) and 2j+2
// (B); at barrier 2m+1 the copies of K_{m+2} (over K_m) and V_{m+1} (over
// V_{m-1}) start, and each wave waits for them before barrier 2m+3. Each
// group runs its own loop; both pass the same number of barriers.
// SYNC = 2 keeps a barrier between every two intervals. SYNC = 1 keeps only
// the odd ones: every LDS read of a block falls between the odd barriers
// around it (K_j in (2j-1, 2j+1), V_j in (2j+1, 2j+3)), so the ring stays
// safe, and the even barrier only enforced the turn change; without it a
// wave that ends its turn early starts the next one instead of waiting.
template <int D, int NW, int BN, int QT, bool CAUSAL, int VS, int KS, typename CopyFn>
__device__ __forceinline__ void pingpong_mfma_turn(const Ctx& c, char* smem, int jp,
                                                   const LdsOffsets<D>& off,
                                                   const bf16x8 (&qf)[QT][D / 16],
                                                   f32x16 (&s)[QT][BN / 32],
                                                   const bf16x8 (&pb)[QT][BN / 16],
                                                   f32x16 (&o)[QT][D / 32], int ncopy, CopyFn&& copy) {
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  // the wave on the matrix core issues ahead of the wave in its softmax turn
  // (measured: +2% over equal priority, -2% with the priorities reversed)
  __builtin_amdgcn_s_setprio(1);
  if (jp >= 0 && jp < c.nblk && jp * BN < c.kv_end_w) {
    pv_block<D, BN, QT>(v_slot<D, BN, 2>(smem, VS), off, pb, o);
    sched_mfma_with_reads<(BN / 16) * (D / 32), 2, QT, kPfPVTurn>();
  }
  const int jq = jp + 1;
  if (jq < c.nblk && jq * BN < c.kv_end_w) {
    if (ncopy)
      qk_block_with_copies<D, BN, QT, 2 * LD>(k_slot<D, BN, 2>(smem, KS), off, qf, s, copy);
    else
      qk_block<D, BN, QT>(k_slot<D, BN, 2>(smem, KS), off, qf, s);
    sched_mfma_with_reads<(D / 16) * (BN / 32), 1, QT, kPfQK>();
  } else if (ncopy) {
#pragma unroll
    for (int ci = 0; ci < 2 * LD; ++ci) copy(ci);
  }
}

// The softmax turn, with NCOPY copy instructions (group B's share of the
// next blocks): half open the turn, half follow the row sums, where the
// texture path has drained the other group's copies (measured +1% over all
// at the start; one after each key tile's exps measured no better).
template <int D, int BN, int QT, bool CAUSAL, int NCOPY, typename CopyFn>
__device__ __forceinline__ void pingpong_valu_turn(const Ctx& c, int j, f32x16 (&s)[QT][BN / 32],
                                                   bf16x8 (&pb)[QT][BN / 16],
                                                   f32x16 (&o)[QT][D / 32], float (&m_run)[QT], float (&ms_run)[QT],
                                                   float (&l_run)[QT], CopyFn&& copy) {
  constexpr int NB = BN / 32;
  __builtin_amdgcn_s_setprio(0);
  if (j < c.nblk && j * BN < c.kv_end_w) {
    const int kv0 = j * BN;
#pragma unroll
    for (int ci = 0; ci < NCOPY / 2; ++ci) copy(ci);
    if (block_needs_mask<BN, CAUSAL>(c, kv0)) mask_block<BN, QT, CAUSAL>(s, kv0, c.qi0, c.N, c.lane);
    float alpha[QT], ps[QT][4];
    softmax_stats<BN, QT>(s, c.c_log2, m_run, ms_run, alpha);
    static_for<NB>([&](auto KB) { softmax_exp<BN, QT, KB>(s, c.c_log2, m_run, ps); });
    softmax_pack<BN, QT>(s, pb);
    softmax_sum<QT>(l_run, alpha, ps);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ci = NCOPY / 2; ci < NCOPY; ++ci) copy(ci);
    __builtin_amdgcn_sched_barrier(0);
    rescale_block<D, QT>(o, alpha);
  } else {
#pragma unroll
    for (int ci = 0; ci < NCOPY; ++ci) copy(ci);
  }
}

// Start of an odd interval t = 2m+1: every wave waits for its share of the
// copies started two intervals ago and meets the others at the barrier; the
// copies of K_{m+2} (over K_m, slot MS) and V_{m+1} (over V_{m-1}, slot MS^1)
// are then issued by the returned functor, spread over the wave's next turn.
// Past the last block a clamped duplicate lands in a slot nobody reads again.
template <int D, int NW, int BN, int MS>
__device__ __forceinline__ auto pingpong_odd_barrier(const Ctx& c, char* smem, int m) {
  wait_vmcnt<0>();
  block_barrier();
  const int row_k = min(m + 2, c.nblk - 1) * BN;
  const int row_v = min(m + 1, c.nblk - 1) * BN;
  return [&c, smem, row_k, row_v](int ci) {
    const int t = ci >> 1;
    if (ci & 1)
      issue_copy<D, NW, BN, true>(c.Vh, row_v, c.N, v_slot<D, BN, 2>(smem, MS ^ 1), c.wave, c.lane, t);
    else
      issue_copy<D, NW, BN, false>(c.Kh, row_k, c.N, k_slot<D, BN, 2>(smem, MS), c.wave, c.lane, t);
  };
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int SYNC>
__device__ __forceinline__ void attn_fwd_pingpong_tile(const Ctx& c, char* smem,
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, 2>;
  static_assert(NW % 2 == 0, "two wave groups");

  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, q_mode, qf, c.lane);
  issue_block_load<D, NW, BN, false>(c.Kh, 0, N, k_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  issue_block_load<D, NW, BN, true>(c.Vh, 0, N, v_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  if (c.nblk > 1)
    issue_block_load<D, NW, BN, false>(c.Kh, BN, N, k_slot<D, BN, 2>(smem, 1), c.wave, c.lane);
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], ms_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
    ms_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }
  f32x16 s[QT][BN / 32];
  bf16x8 pb[QT][BN / 16];
  wait_vmcnt<0>();
  block_barrier();
  const int n = c.nblk;
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  auto no_copy = [](int) {};
  // Both groups pass 2n+1 barriers after the prologue one.
  if (c.wave < NW / 2) {
    qk_block<D, BN, QT>(k_slot<D, BN, 2>(smem, 0), off, qf, s);  // S_0 (block 0 is never skipped)
    sched_mfma_with_reads<(D / 16) * (BN / 32), 1, QT, kPfQK>();
    for (int j = 0; j < n; j += 2) {
      // block j (even): [t=2j] softmax | [t=2j+1] pv(j) from V slot 0, qk(j+1) from K slot 1
      if constexpr (SYNC == 2) block_barrier();
      pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j, s, pb, o, m_run, ms_run, l_run, no_copy);
      {
        auto copy = pingpong_odd_barrier<D, NW, BN, 0>(c, smem, j);
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, j, off, qf, s, pb, o, 1, copy);
      }
      if (j + 1 < n) {  // block j+1 (odd): slots swap
        if constexpr (SYNC == 2) block_barrier();
        pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j + 1, s, pb, o, m_run, ms_run, l_run, no_copy);
        auto copy = pingpong_odd_barrier<D, NW, BN, 1>(c, smem, j + 1);
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, j + 1, off, qf, s, pb, o, 1, copy);
      }
    }
    block_barrier();  // t = 2n: group B's last mma_pv
  } else {
    for (int j = 0; j < n; j += 2) {
      // block j (even): [t=2j] pv(j-1) from V slot 1, qk(j) from K slot 0 | [t=2j+1] softmax
      if constexpr (SYNC == 2) block_barrier();
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, j - 1, off, qf, s, pb, o, 0, no_copy);
      {
        auto copy = pingpong_odd_barrier<D, NW, BN, 0>(c, smem, j);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j, s, pb, o, m_run, ms_run, l_run, copy);
      }
      if (j + 1 < n) {
        if constexpr (SYNC == 2) block_barrier();
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, j, off, qf, s, pb, o, 0, no_copy);
        auto copy = pingpong_odd_barrier<D, NW, BN, 1>(c, smem, j + 1);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j + 1, s, pb, o, m_run, ms_run, l_run, copy);
      }
    }
    block_barrier();  // t = 2n: mma_pv of the last block, from V slot (n-1) & 1
    if (n & 1)
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, n - 1, off, qf, s, pb, o, 0, no_copy);
    else
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, n - 1, off, qf, s, pb, o, 0, no_copy);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, ms_run, l_run, c.c_log2, c.lane);
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int SYNC>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_pingpong(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, 2>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  if constexpr (!CAUSAL) {
    Ctx c;
    make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, 0, c);
    attn_fwd_pingpong_tile<D, NW, BN, QT, CAUSAL, OCC, SYNC>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
  } else {
    for (int pass = 0; pass < 2; ++pass) {
      Ctx c;
      if (!make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, pass, c)) break;
      if (pass > 0) block_barrier();  // every wave is done with the ring of the previous tile
      attn_fwd_pingpong_tile<D, NW, BN, QT, CAUSAL, OCC, SYNC>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
    }
  }
}

// ---------------------------------------------------------------- fused ping-pong kernel
// The ping-pong schedule above with every matrix turn as one fused stream
// (fused_pv_qk: the K^T reads of mma_qk start during the last mma_pv MFMAs).
// So that the loop has a single code path (one register assignment, no
// copies of O between paths), every turn of a wave up to its last live block
// takes the fused stream: group B's first turn multiplies zeros (P = 0 and a
// zero-filled V slot, O stays +0 exactly), and a wave's last turn computes a
// QK^T product that is never used (its K slot always holds finite data: a
// later block, or a clamped duplicate of the last one). Turns past a wave's
// last live block are skipped whole. Intervals, slots, copies and barriers
// are the ping-pong kernel's.
//
// PRE = 1: group B also reads the first V fragment pairs of its next matrix
// turn at the end of its softmax turn (those V rows were certified by the
// barrier that opened the softmax turn); its copies then go through inline
// assembly, which keeps the compiler from draining them before the
// transposing reads (every wait on them is the explicit one before the odd
// barriers).
template <int D, int NW, int BN, int MS, bool ASM>
__device__ __forceinline__ auto pp_odd_barrier(const Ctx& c, char* smem, int m) {
  wait_vmcnt<0>();
  block_barrier();
  const int row_k = min(m + 2, c.nblk - 1) * BN;
  const int row_v = min(m + 1, c.nblk - 1) * BN;
  return [&c, smem, row_k, row_v](int ci) {
    const int t = ci >> 1;
    if constexpr (ASM) {
      if (ci & 1)
        issue_copy_asm<D, NW, BN, true>(c.Vh, row_v, c.N, v_slot<D, BN, 2>(smem, MS ^ 1), c.wave, c.lane, t);
      else
        issue_copy_asm<D, NW, BN, false>(c.Kh, row_k, c.N, k_slot<D, BN, 2>(smem, MS), c.wave, c.lane, t);
    } else {
      if (ci & 1)
        issue_copy<D, NW, BN, true>(c.Vh, row_v, c.N, v_slot<D, BN, 2>(smem, MS ^ 1), c.wave, c.lane, t);
      else
        issue_copy<D, NW, BN, false>(c.Kh, row_k, c.N, k_slot<D, BN, 2>(smem, MS), c.wave, c.lane, t);
    }
  };
}

// Matrix turn jp: mma_pv(V_jp, slot VS) and mma_qk(K_jp+1, slot KS) as one
// stream when jp is below the wave's live-block count nw; else only the copies.
template <int D, int NW, int BN, int QT, int VS, int KS, int NPRE, int NC, int NPA, typename CopyFn>
__device__ __forceinline__ void pp_fused_matrix_turn(char* smem, int jp, int nw, const LdsOffsets<D>& off,
                                                     const bf16x8 (&qf)[QT][D / 16], f32x16 (&s)[QT][BN / 32],
                                                     const bf16x8 (&pb)[QT][BN / 16], f32x16 (&o)[QT][D / 32],
                                                     const i16x4 (&pre)[NPA][2], CopyFn&& copy) {
  __builtin_amdgcn_s_setprio(1);
  if (jp < nw) {
    fused_pv_qk<D, BN, QT, NPRE, NC>(v_slot<D, BN, 2>(smem, VS), k_slot<D, BN, 2>(smem, KS), off, qf, s, pb, o,
                                     pre, copy);
  } else {
#pragma unroll
    for (int ci = 0; ci < NC; ++ci) copy(ci);
  }
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int PRE>
__device__ __forceinline__ void attn_fwd_pingpong_fused_tile(const Ctx& c, char* smem,
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, 2>;
  static_assert(NW % 2 == 0, "two wave groups");
  constexpr int NPRE = PRE ? 2 : 0;
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  const int nw = (c.kv_end_w + BN - 1) / BN;  // this wave's live blocks (wave-uniform)

  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, q_mode, qf, c.lane);
  issue_block_load<D, NW, BN, false>(c.Kh, 0, N, k_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  issue_block_load<D, NW, BN, true>(c.Vh, 0, N, v_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  if (c.nblk > 1)
    issue_block_load<D, NW, BN, false>(c.Kh, BN, N, k_slot<D, BN, 2>(smem, 1), c.wave, c.lane);
  {
    // zero V slot 1 for group B's first (all-zero) P.V
    char* v1 = v_slot<D, BN, 2>(smem, 1);
    constexpr int PER = BN * D * 2 / (NW * 64 * 16);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      *(LDS_AS u32x4*)(v1 + ((i * NW + c.wave) * 64 + c.lane) * 16) = u32x4{0, 0, 0, 0};
  }
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], ms_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
    ms_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }
  f32x16 s[QT][BN / 32];
  bf16x8 pb[QT][BN / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int p = 0; p < BN / 16; ++p) pb[qt][p] = bf16x8{};
  i16x4 pre[NPRE > 0 ? NPRE : 1][2];
#pragma unroll
  for (int g = 0; g < (NPRE > 0 ? NPRE : 1); ++g) pre[g][0] = pre[g][1] = i16x4{0, 0, 0, 0};
  wait_vmcnt<0>();
  block_barrier();
  const int n = c.nblk;
  auto no_copy = [](int) {};
  // Both groups pass 2n+1 barriers after the prologue one.
  if (c.wave < NW / 2) {
    qk_block<D, BN, QT>(k_slot<D, BN, 2>(smem, 0), off, qf, s);  // S_0 (block 0 is never skipped)
    sched_mfma_with_reads<(D / 16) * (BN / 32), 1, QT, kPfQK>();
    for (int j = 0; j < n; j += 2) {
      // block j (even): [t=2j] softmax | [t=2j+1] pv(j) from V slot 0, qk(j+1) from K slot 1
      block_barrier();
      pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j, s, pb, o, m_run, ms_run, l_run, no_copy);
      {
        auto copy = pp_odd_barrier<D, NW, BN, 0, false>(c, smem, j);
        pp_fused_matrix_turn<D, NW, BN, QT, 0, 1, 0, 2 * LD>(smem, j, nw, off, qf, s, pb, o, pre, copy);
      }
      if (j + 1 < n) {  // block j+1 (odd): slots swap
        block_barrier();
        pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j + 1, s, pb, o, m_run, ms_run, l_run, no_copy);
        auto copy = pp_odd_barrier<D, NW, BN, 1, false>(c, smem, j + 1);
        pp_fused_matrix_turn<D, NW, BN, QT, 1, 0, 0, 2 * LD>(smem, j + 1, nw, off, qf, s, pb, o, pre, copy);
      }
    }
    block_barrier();  // t = 2n: group B's last mma_pv
  } else {
    for (int j = 0; j < n; j += 2) {
      // block j (even): [t=2j] pv(j-1) from V slot 1, qk(j) from K slot 0 | [t=2j+1] softmax
      block_barrier();
      pp_fused_matrix_turn<D, NW, BN, QT, 1, 0, NPRE, 0>(smem, j - 1, nw, off, qf, s, pb, o, pre, no_copy);
      {
        auto copy = pp_odd_barrier<D, NW, BN, 0, PRE != 0>(c, smem, j);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j, s, pb, o, m_run, ms_run, l_run, copy);
        if constexpr (NPRE > 0) {
          if (j < nw) static_for<NPRE>([&](auto G) { read_v_pair<D, G>(v_slot<D, BN, 2>(smem, 0), off, pre[G]); });
        }
      }
      if (j + 1 < n) {
        block_barrier();
        pp_fused_matrix_turn<D, NW, BN, QT, 0, 1, NPRE, 0>(smem, j, nw, off, qf, s, pb, o, pre, no_copy);
        auto copy = pp_odd_barrier<D, NW, BN, 1, PRE != 0>(c, smem, j + 1);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j + 1, s, pb, o, m_run, ms_run, l_run, copy);
        if constexpr (NPRE > 0) {
          if (j + 1 < nw)
            static_for<NPRE>([&](auto G) { read_v_pair<D, G>(v_slot<D, BN, 2>(smem, 1), off, pre[G]); });
        }
      }
    }
    block_barrier();  // t = 2n: mma_pv of the last block, from V slot (n-1) & 1
    if (n & 1)
      pp_fused_matrix_turn<D, NW, BN, QT, 0, 1, NPRE, 0>(smem, n - 1, nw, off, qf, s, pb, o, pre, no_copy);
    else
      pp_fused_matrix_turn<D, NW, BN, QT, 1, 0, NPRE, 0>(smem, n - 1, nw, off, qf, s, pb, o, pre, no_copy);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, ms_run, l_run, c.c_log2, c.lane);
}

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC, int PRE>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_pingpong_fused(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int q_mode) {
  using T = Tile<D, NW, BN, QT, 2>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  if constexpr (!CAUSAL) {
    Ctx c;
    make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, 0, c);
    attn_fwd_pingpong_fused_tile<D, NW, BN, QT, CAUSAL, OCC, PRE>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
  } else {
    for (int pass = 0; pass < 2; ++pass) {
      Ctx c;
      if (!make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2, pass, c)) break;
      if (pass > 0) block_barrier();  // every wave is done with the ring of the previous tile
      attn_fwd_pingpong_fused_tile<D, NW, BN, QT, CAUSAL, OCC, PRE>(c, smem, Q, K, V, O, LSE, N, n_qtiles, c_log2, q_mode);
    }
  }
}

}  // namespace

#endif  // ATTN_FWD_KERNELS_H
