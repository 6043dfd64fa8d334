// attn_common.h -- device-side building blocks shared by the kernels of
// libattn.so (one copy per translation unit, internal linkage): vector
// types, the LDS swizzles and HBM -> LDS copies, the per-block steps of the
// attention forward (mma_qk, mask, online softmax, rescale, mma_pv, store),
// the workgroup barrier and explicit copy waits. The forward kernels, the
// split-KV decoding, the backward, Mamba2 ChunkScan and MLA decoding each
// live in their own .hip file and include this header.
#ifndef ATTN_COMMON_H
#define ATTN_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so
// register arrays are only ever indexed by constants (never spilled to
// scratch by a partially unrolled loop).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

// NW waves, QT query tiles of 32 per wave, BN keys per block, ST ring slots.
template <int D, int NW, int BN, int QT = 1, int ST = 2>
struct Tile {
  static constexpr int BM = 32 * QT * NW;            // query rows per workgroup
  static constexpr int RC = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int MAT_BYTES = BN * D * 2;       // one K (or V) block in LDS
  static constexpr int STAGE_BYTES = 2 * MAT_BYTES;  // K + V
  static constexpr int LDS_BYTES = ST * STAGE_BYTES; // ring of ST stages
  static constexpr int LOADS = MAT_BYTES / (16 * 64 * NW);  // 1 KiB wave copies per matrix
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BN % 32 == 0, "BN multiple of 32");
  static_assert(LOADS * 16 * 64 * NW == MAT_BYTES, "block must split evenly over waves");
  static_assert(ST >= 2, "at least double buffering");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

// Row swizzles of the LDS images (chunk = 16 bytes). K rows are read 16
// rows at a time at one chunk column (ds_read_b128): XOR with the row index
// spreads them over all banks. V rows are read by ds_read_b64_tr_b16 in
// groups of 4 consecutive rows x 32 bytes: XOR with 4*(row mod 4) (pairs of
// chunks stay together) puts the 4 rows on distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 64 ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
}
// For an image read both ways (row fragments and transposed reads, as the
// backward's Q, dO and K images are): a permutation of the 16 chunk columns
// over 16 consecutive rows (row fragments conflict-free, as swz_k) whose bits
// 2-3 differ between the 4 rows of every aligned group (transposed reads
// conflict-free, as swz_v). At d = 64 a 256-byte bank line holds two rows,
// so the same holds per row pair.
template <int D>
__device__ __forceinline__ int swz_dual(int row) {
  return D == 64 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : (((row & 3) << 2) | ((row >> 2) & 3));
}

// HBM -> LDS copies of BN-row blocks of one [N][D] matrix. Every wave moves
// LOADS x 1 KiB per block; lane l's 16 bytes land at dst + 16*l, so the
// swizzle is applied by choosing the source chunk. The source is a buffer
// resource over rows [row0, min(row0 + BN, N)): the hardware range check
// turns reads of rows past N into zeros (those keys are masked and their
// weights are exactly zero), so a copy needs no per-lane address arithmetic
// beyond its fixed lane offset.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// Swizzle kinds: 0 = swz_k, 1 = swz_v, 2 = swz_dual.
template <int D, int SW>
__device__ __forceinline__ int swz(int row) {
  return SW == 0 ? swz_k<D>(row) : SW == 1 ? swz_v<D>(row) : swz_dual<D>(row);
}

template <int D, int NW, int BN, int SW>
__device__ __forceinline__ uint32_t block_lane_offset_sw(int t, int wave, int lane) {
  using T = Tile<D, NW, BN>;
  const int p = (t * NW + wave) * 64 + lane;
  const int row = p / T::RC;
  const int pc = p % T::RC;
  const int c = pc ^ swz<D, SW>(row);
  return (uint32_t)(row * (D * 2) + c * 16);
}
template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ uint32_t block_lane_offset(int t, int wave, int lane) {
  return block_lane_offset_sw<D, NW, BN, IS_V ? 1 : 0>(t, wave, lane);
}

// row0 < N always (callers clamp block indices to the last block). The byte
// count is made explicitly wave-uniform: a min/max clamp otherwise becomes a
// VALU med3 and the resource a per-lane value.
template <int D, int BN>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* src, int row0, int N) {
  const int rows = __builtin_amdgcn_readfirstlane(min(N - row0, BN));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)row0 * D), (short)0, rows * (D * 2),
                                           kRsrcWord3);
}

// Copy instruction t of the block at row0.
template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ void issue_copy(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                           int wave, int lane, int t) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc<D, BN>(src, row0, N);
  const int off = (int)block_lane_offset<D, NW, BN, IS_V>(t, wave, lane);
  LDS_AS void* to = (LDS_AS void*)(dst + (t * NW + wave) * 64 * 16);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to, 16, off, 0, 0, 0);
}

// All copy instructions of the block at row0.
template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ void issue_block_load(const uint16_t* __restrict__ src, int row0, int N,
                                                 char* dst, int wave, int lane) {
#pragma unroll
  for (int t = 0; t < Tile<D, NW, BN>::LOADS; ++t) issue_copy<D, NW, BN, IS_V>(src, row0, N, dst, wave, lane, t);
}

__device__ __forceinline__ float swap32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> logical tile id. The dispatcher deals workgroups to the 8
// XCDs round-robin; this makes each XCD's share a contiguous logical range.
__device__ __forceinline__ int xcd_remap(int i, int G) {
  const int q = G / 8, r = G % 8;
  const int x = i % 8, k = i / 8;
  return x * q + min(x, r) + k;
}

// ---------------------------------------------------------------- per-block steps
// Each helper is one step of the per-block schedule; all kernels call the
// same helpers in the same per-block order, so their results agree bit for
// bit and differ only in how steps overlap.

// Per-lane LDS byte offsets of the MFMA operand fragments within one K (or
// V) block image. They depend only on the lane, so they are computed once;
// the key-tile, half and ring-slot offsets are compile-time immediates.
template <int D>
struct LdsOffsets {
  int k[D / 16];  // K fragment for d-chunk kk: row lq, 16-byte chunk 2kk+h
  int v[D / 32];  // V^T transposed read for dim tile t (first of the 8-row pair)
  __device__ __forceinline__ explicit LdsOffsets(int lane) {
    const int h = lane >> 5, lq = lane & 31, ci = lane & 15, g2 = (lane >> 4) & 1;
    const int swk = swz_k<D>(lq);  // equal for rows lq + 32*kb
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k[kk] = lq * (D * 2) + (((2 * kk + h) ^ swk) << 4);
    const int r0 = 4 * h + (ci >> 2);  // + 32*kb + 16*hf + 8*pair: swizzle-neutral offsets
    const int swv = swz_v<D>(r0);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int dd = t * 32 + g2 * 16 + 4 * (ci & 3);
      v[t] = r0 * (D * 2) + (((dd >> 3) ^ swv) << 4) + (dd & 7) * 2;
    }
  }
};

// Scheduling patterns (sched_group_barrier masks: 0x008 MFMA, 0x100 DS
// read, 0x002 VALU). Reads run PF reads ahead of the MFMAs that consume them;
// each read feeds MR MFMAs.
template <int NR, int RD, int MR, int PF>
__device__ __forceinline__ void sched_mfma_with_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, RD * PF, 0);
#pragma unroll
  for (int i = 0; i < NR - PF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MR, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MR * PF, 0);
}

// Pin a value's computation before this point (an empty asm that "uses" it):
// keeps the compiler from sinking overlapped softmax work out of the MFMA
// stream it was scheduled into.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Copies interleaved with an MFMA stream of NR read groups whose reads run PF
// groups ahead: copy c of NC is issued in steady step (c * (NR - PF)) / NC,
// right after that step's reads (read group PF + step); a stream with no
// steady part (NR <= PF) issues them all after its last read. The stream's
// program order and its scheduling pattern both use this placement, so the
// compiler (which keeps LDS-writing copies and LDS reads in order) can honour
// both.
template <int NR, int PF, int NC>
constexpr int copy_step(int c) {
  return NC > 0 ? (c * (NR - PF)) / NC : 0;
}
template <int NR, int PF, int NC>
constexpr int copy_after_group(int c) {
  return NR > PF ? PF + copy_step<NR, PF, NC>(c) : NR - 1;
}
template <int NR, int PF, int NC>
constexpr int copies_due(int step) {
  int n = 0;
  for (int c = 0; c < NC; ++c) n += copy_step<NR, PF, NC>(c) == step;
  return n;
}

// With one wave per SIMD a wave has 256 VGPRs plus 256 AGPRs. The Q^T
// fragments are only ever MFMA B operands, which may come from AGPRs, so they
// are parked there; this keeps O (which the rescale updates on the VALU) in
// VGPRs. Left alone, the compiler parks O in AGPRs instead and moves it out
// and back every block (about 2 x d/2 v_accvgpr moves per block at d = 256).
template <int QT, int ND>
__device__ __forceinline__ void park_in_agprs(bf16x8 (&qf)[QT][ND]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kk = 0; kk < ND; ++kk) asm volatile("" : "=a"(qf[qt][kk]) : "0"(qf[qt][kk]));
}

constexpr int kPfQK = 4;  // K fragments in flight ahead of mma_qk
constexpr int kPfPV = 2;  // V fragment pairs in flight ahead of mma_pv
constexpr int kPfPVTurn = 3;  // the same for a ping-pong matrix turn (one wave streams alone)

// mma_qk: S^T[key][query] for BN keys (K block image at Ks) against the
// wave's QT query tiles. A operand = K rows (ds_read_b128), B operand = Q^T.
// All fragment reads are issued up front in program order; the caller's
// scheduling pattern places them ahead of their MFMAs.
template <int D, int BN, int QT>
__device__ __forceinline__ void qk_block(const char* Ks, const LdsOffsets<D>& off,
                                         const bf16x8 (&qf)[QT][D / 16],
                                         f32x16 (&s)[QT][BN / 32]) {
  constexpr int NKB = BN / 32;
  bf16x8 kf[D / 16][NKB];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      kf[kk][kb] = *(LDS_AS const bf16x8*)(Ks + off.k[kk] + kb * 32 * (D * 2));
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[qt][kb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        s[qt][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][kb], qf[qt][kk], s[qt][kb], 0, 0, 0);
}

// mma_qk with NCOPY copy instructions of a later block placed between the
// fragment reads in program order at the copy_step positions, spreading the
// texture-path work over the MFMA stream instead of bursting it after the
// barrier.
template <int D, int BN, int QT, int NCOPY, typename CopyFn>
__device__ __forceinline__ void qk_block_with_copies(const char* Ks, const LdsOffsets<D>& off,
                                                     const bf16x8 (&qf)[QT][D / 16],
                                                     f32x16 (&s)[QT][BN / 32], CopyFn&& copy) {
  constexpr int NKB = BN / 32;
  constexpr int NQ = (D / 16) * NKB;
  bf16x8 kf[D / 16][NKB];
  static_for<NQ>([&](auto I) {
    constexpr int i = I;
    kf[i / NKB][i % NKB] = *(LDS_AS const bf16x8*)(Ks + off.k[i / NKB] + (i % NKB) * 32 * (D * 2));
    static_for<NCOPY>([&](auto C) {
      static_assert(copy_after_group<NQ, kPfQK, NCOPY>(C) < NQ, "every copy is placed");
      if constexpr (copy_after_group<NQ, kPfQK, NCOPY>(C) == i) copy(int(C));
    });
  });
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[qt][kb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        s[qt][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][kb], qf[qt][kk], s[qt][kb], 0, 0, 0);
}

// Masked pairs (key past N, or key after the query when causal) get -inf.
// qi0 = this lane's query in tile 0; tile qt holds queries qi0 + 32*qt.
template <int BN, int QT, bool CAUSAL>
__device__ __forceinline__ void mask_block(f32x16 (&s)[QT][BN / 32], int kv0, int qi0, int N,
                                           int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const bool dead = (key >= N) || (CAUSAL && key > qi0 + 32 * qt);
        s[qt][kb][r] = dead ? -INFINITY : s[qt][kb][r];
      }
}

// softmax (per query tile), in three pieces so that overlapped schedules can
// spread it over MFMA streams; every schedule runs the same pieces in the
// same order, so results agree bit for bit:
//   softmax_stats: new running max (exact: max has no rounding, so the order
//                  of the max tree is free), alpha = exp2(m_old - m_new)
//                  (1 exactly when the max did not move, 0 on the first
//                  block);
//   softmax_exp<KB>: p = exp2(c*s - m) for key tile KB, written over the
//                  scores, with the row sum taken from fp32 p (tile 0 first,
//                  registers in order);
//   softmax_pack:  P^T to bf16 (RNE) as the B operand of mma_pv:
//                  pb[qt][2*kb + hf] holds accumulator registers 8*hf..8*hf+7
//                  of key tile kb;
//   softmax_sum:   l = l * alpha + (ps0 + ps1) + (ps2 + ps3).
//   ms_run (the overloads that take it): the running max of the unscaled
//                  scores, which the epilogue needs to recover the dominant
//                  key's fp32 weight (store_rows).
template <int BN, int QT>
__device__ __forceinline__ void softmax_stats(const f32x16 (&s)[QT][BN / 32], float c_log2,
                                              float (&m_run)[QT], float (&ms_run)[QT], float (&alpha)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // four left-deep chains over the lane's 16 * BN/32 scores, written so
    // that each step folds two new scores (one v_max3_f32); pairwise maxima
    // would cost 1.5x the instructions
    constexpr int NCH = 4, NV = 16 * (BN / 32) / NCH;
    static_assert(NV >= 3 && NV % 2 == 0, "chain length");
    float mx[NCH];
#pragma unroll
    for (int h2 = 0; h2 < NCH; ++h2) {
      auto v = [&](int i) { const int g = h2 * NV + i; return s[qt][g / 16][g % 16]; };
      float m = fmaxf(fmaxf(v(0), v(1)), v(2));
#pragma unroll
      for (int i = 3; i + 1 < NV; i += 2) m = fmaxf(fmaxf(m, v(i)), v(i + 1));
      mx[h2] = fmaxf(m, v(NV - 1));
    }
    const float bmax = swap32_max(fmaxf(fmaxf(fmaxf(mx[0], mx[1]), mx[2]), mx[3]));
    // c > 0, so fl(max(s) c) = max(fl(s c)): m_run is the max of the scaled scores
    const float m_new = fmaxf(m_run[qt], bmax * c_log2);
    alpha[qt] = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
    m_run[qt] = m_new;
    ms_run[qt] = fmaxf(ms_run[qt], bmax);
  }
}
template <int BN, int QT>
__device__ __forceinline__ void softmax_stats(const f32x16 (&s)[QT][BN / 32], float c_log2,
                                              float (&m_run)[QT], float (&alpha)[QT]) {
  float ms[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) ms[qt] = -INFINITY;
  softmax_stats<BN, QT>(s, c_log2, m_run, ms, alpha);
}

template <int BN, int QT, int KB>
__device__ __forceinline__ void softmax_exp(f32x16 (&s)[QT][BN / 32], float c_log2,
                                            const float (&m_run)[QT], float (&ps)[QT][4]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][KB][r], c_log2, -m_run[qt]));
      s[qt][KB][r] = p;  // in place: the score is dead once its weight exists
      // the first four terms start the four partial sums (0 + p == p exactly)
      if (KB == 0 && r < 4) ps[qt][r] = p;
      else ps[qt][r & 3] += p;
    }
}

template <int BN, int QT>
__device__ __forceinline__ void softmax_pack(const f32x16 (&s)[QT][BN / 32], bf16x8 (&pb)[QT][BN / 16]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      pb[qt][2 * kb] = __builtin_convertvector(
          __builtin_shufflevector(s[qt][kb], s[qt][kb], 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
      pb[qt][2 * kb + 1] = __builtin_convertvector(
          __builtin_shufflevector(s[qt][kb], s[qt][kb], 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
    }
}

template <int QT>
__device__ __forceinline__ void softmax_sum(float (&l_run)[QT], const float (&alpha)[QT],
                                            const float (&ps)[QT][4]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    l_run[qt] = __builtin_fmaf(l_run[qt], alpha[qt], (ps[qt][0] + ps[qt][1]) + (ps[qt][2] + ps[qt][3]));
}

// All of softmax for one block; S is overwritten with P (fp32).
template <int BN, int QT>
__device__ __forceinline__ void softmax_block(f32x16 (&s)[QT][BN / 32], bf16x8 (&pb)[QT][BN / 16],
                                              float c_log2, float (&m_run)[QT], float (&ms_run)[QT],
                                              float (&l_run)[QT], float (&alpha)[QT]) {
  float ps[QT][4];
  softmax_stats<BN, QT>(s, c_log2, m_run, ms_run, alpha);
  static_for<BN / 32>([&](auto KB) { softmax_exp<BN, QT, KB>(s, c_log2, m_run, ps); });
  softmax_pack<BN, QT>(s, pb);
  softmax_sum<QT>(l_run, alpha, ps);
}
template <int BN, int QT>
__device__ __forceinline__ void softmax_block(f32x16 (&s)[QT][BN / 32], bf16x8 (&pb)[QT][BN / 16],
                                              float c_log2, float (&m_run)[QT], float (&l_run)[QT],
                                              float (&alpha)[QT]) {
  float ms[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) ms[qt] = -INFINITY;
  softmax_block<BN, QT>(s, pb, c_log2, m_run, ms, l_run, alpha);
}

// rescale: O *= alpha, per query tile, skipped by the whole wave when no row
// of the tile moved its max.
template <int D, int QT>
__device__ __forceinline__ void rescale_block(f32x16 (&o)[QT][D / 32], const float (&alpha)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    if (__builtin_amdgcn_ballot_w64(alpha[qt] != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) o[qt][t] *= alpha[qt];
    }
}

// mma_pv: O^T[dim][query] += V^T[dim][key] P^T[key][query]. The A operand
// holds, for dim row t*32 + (lane & 31), the same 8 keys as this lane's half
// of the B operand (keys kb*32 + 16*hf + 4*h + {0..3, 8..11}), read as two
// 4-key transposed loads (ds_read_b64_tr_b16) 8 rows apart; each V fragment
// feeds QT MFMAs.
template <int D, int BN, int QT>
__device__ __forceinline__ void pv_block(const char* Vs, const LdsOffsets<D>& off,
                                         const bf16x8 (&pb)[QT][BN / 16],
                                         f32x16 (&o)[QT][D / 32]) {
  constexpr int NP = BN / 16;
  i16x4 va[NP][D / 32][2];
#pragma unroll
  for (int p = 0; p < NP; ++p)  // p = 2*kb + hf: rows p*16 + ...
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        va[p][t][r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(Vs + off.v[t] + (p * 16 + r * 8) * (D * 2)));
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[p][t][0], va[p][t][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        o[qt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qt][p], o[qt][t], 0, 0, 0);
    }
}

// How every kernel takes the scale: the exponent multiplier c = |scale| log2(e)
// is positive (so -inf masks stay -inf and the max is taken on unscaled
// scores), and the sign goes into the operand held in registers, q_mode:
// 0 = as stored, 1 = every sign bit flipped (a negative scale; exact in
// bf16), 2 = zeros (a zero scale makes every logit exactly 0, which a zero
// operand with c = log2(e) reproduces exactly).
struct ScaleArgs {
  float c_log2;
  int q_mode;
};
__host__ __device__ inline ScaleArgs scale_args(float scale) {
  if (scale == 0.f) return ScaleArgs{kLog2e, 2};
  return ScaleArgs{fabsf(scale) * kLog2e, scale < 0.f ? 1 : 0};
}

// HIP keeps one "last error" per host thread, set by any failing runtime call
// (the caller's included). Entry points clear it right before their launches,
// so that the hipGetLastError after them reports those launches only.
inline void clear_last_hip_error() { (void)hipGetLastError(); }

// 8 bf16 values as q_mode asks (see scale_args).
__device__ __forceinline__ u32x4 apply_q_mode(u32x4 raw, int q_mode) {
  if (q_mode == 1) raw ^= 0x80008000u;  // exact sign flip of 8 bf16 values
  if (q_mode == 2) raw = u32x4{0u, 0u, 0u, 0u};
  return raw;
}

// Load the wave's Q^T fragments (B operand of mma_qk): lane holds
// Q[q][kk*16 + h*8 .. +7] for its query q of each tile (rows past N clamped),
// taken as q_mode asks.
template <int D, int QT>
__device__ __forceinline__ void load_q(const uint16_t* Qh, int q0w, int N, int q_mode,
                                       bf16x8 (&qf)[QT][D / 16], int lane) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qrow = min(q0w + 32 * qt + (lane & 31), N - 1);
    const uint16_t* qp = Qh + (size_t)qrow * D + (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[qt][kk] = __builtin_bit_cast(bf16x8, apply_q_mode(*(const u32x4*)(qp + kk * 16), q_mode));
  }
}

// Epilogue: O = O_acc / l and LSE = ln2 * (m + log2 l), stored for rows < N.
// With ms_run (the unscaled running max) O is normalised by l with the
// dominant key's weight taken as the matrix core used it: that weight is
// exp2 of the exponent argument's fp32 residual fma(s_max, c, -fl(s_max c)),
// within 2^-19 of 1 in fp32 (what l holds) and exactly 1 in bf16 (what O_acc
// holds). So a row whose softmax is one-hot up to fp32 (causal row 0, a key
// far above the others) stores exactly its dominant V row. LSE uses l.
template <int D, int QT, bool DOM>
__device__ __forceinline__ void store_rows_impl(float* O, float* LSE, size_t head, size_t bh, int N,
                                                int qi0, const f32x16 (&o)[QT][D / 32],
                                                const float (&m_run)[QT], const float (&ms_run)[QT],
                                                const float (&l_run)[QT], float c_log2, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = qi0 + 32 * qt;
    const float l_tot = swap32_sum(l_run[qt]);
    float l_o = l_tot;
    if constexpr (DOM) {
      const float p_dom = __builtin_amdgcn_exp2f(__builtin_fmaf(ms_run[qt], c_log2, -m_run[qt]));
      l_o = (l_tot - p_dom) + 1.0f;
    }
    const float inv = 1.0f / l_o;
    if (qi < N) {
      float* orow = O + head + (size_t)qi * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w = {o[qt][t][4 * g] * inv, o[qt][t][4 * g + 1] * inv, o[qt][t][4 * g + 2] * inv,
                     o[qt][t][4 * g + 3] * inv};
          *(f32x4*)(orow + t * 32 + g * 8 + h * 4) = w;
        }
      if (h == 0) LSE[bh * N + qi] = kLn2 * (m_run[qt] + __builtin_amdgcn_logf(l_tot));
    }
  }
}
template <int D, int QT>
__device__ __forceinline__ void store_rows(float* O, float* LSE, size_t head, size_t bh, int N, int qi0,
                                           const f32x16 (&o)[QT][D / 32], const float (&m_run)[QT],
                                           const float (&ms_run)[QT], const float (&l_run)[QT], float c_log2,
                                           int lane) {
  store_rows_impl<D, QT, true>(O, LSE, head, bh, N, qi0, o, m_run, ms_run, l_run, c_log2, lane);
}
template <int D, int QT>
__device__ __forceinline__ void store_rows(float* O, float* LSE, size_t head, size_t bh, int N, int qi0,
                                           const f32x16 (&o)[QT][D / 32], const float (&m_run)[QT],
                                           const float (&l_run)[QT], int lane) {
  store_rows_impl<D, QT, false>(O, LSE, head, bh, N, qi0, o, m_run, m_run, l_run, 0.f, lane);
}

// Everything a block step needs besides the per-block registers.
struct Ctx {
  const uint16_t* Kh;
  const uint16_t* Vh;
  size_t head;
  int bh;
  int N, nblk, kv_end_w, q0, q0w, qi0, wave, lane;
  float c_log2;
};

// Workgroup -> (batch*head, query tile) and the per-wave key range, for pass
// `pass` of the workgroup. Without a mask every query tile costs the same and
// a workgroup takes one. With the causal mask tile t costs t+1 units, so a
// workgroup takes two: tile n-1-p, then tile p (one when they coincide), and
// every workgroup gets the same n+1 units: the grid is one balanced round
// instead of long tiles finishing late. The ids of one head are contiguous in
// the XCD-remapped order, so its K/V stays in one XCD's L2. Returns false
// when the workgroup has no tile for this pass (wave-uniform).
template <int D, int BM, int BN, int WROWS, bool CAUSAL>
__device__ __forceinline__ bool make_ctx(const uint16_t* K, const uint16_t* V, int N, int n_qtiles,
                                         float c_log2, int pass, Ctx& c) {
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int tile;
  if (CAUSAL) {
    const int np = (n_qtiles + 1) / 2;  // workgroups per head
    c.bh = L / np;
    const int p = L % np, heavy = n_qtiles - 1 - p;
    if (pass == 0) {
      tile = heavy;
    } else {
      if (p == heavy) return false;
      tile = p;
    }
  } else {
    if (pass > 0) return false;
    c.bh = L / n_qtiles;
    tile = L % n_qtiles;
  }
  const int q0 = tile * BM;
  c.q0 = q0;
  c.q0w = q0 + c.wave * WROWS;
  c.qi0 = c.q0w + (c.lane & 31);
  c.head = (size_t)c.bh * N * D;
  c.Kh = K + c.head;
  c.Vh = V + c.head;
  c.N = N;
  const int kv_end_wg = CAUSAL ? min(N, q0 + BM) : N;
  c.kv_end_w = CAUSAL ? min(N, c.q0w + WROWS) : N;
  c.nblk = (kv_end_wg + BN - 1) / BN;
  c.c_log2 = c_log2;
  return true;
}

// Workgroups in the grid of a forward launch (see make_ctx).
// A dispatch counts its work-items in 32 bits: workgroups times threads per
// workgroup must stay below 2^32 (shapes beyond that are ATTN_ERR_BAD_SHAPE).
inline bool grid_fits(long long workgroups, int threads) { return workgroups <= 0xFFFFFFFFLL / threads; }

__host__ __device__ inline long long fwd_grid(long long BH, int n_qtiles, int causal) {
  return BH * (causal ? (n_qtiles + 1) / 2 : n_qtiles);
}

// Does block j straddle the diagonal (first query of the wave) or the end of K?
template <int BN, bool CAUSAL>
__device__ __forceinline__ bool block_needs_mask(const Ctx& c, int kv0) {
  return (kv0 + BN > c.N) || (CAUSAL && kv0 + BN - 1 > c.q0w);
}

// LDS images of an ST-slot ring: K slot s at s*MAT, V slot s at (ST+s)*MAT.
template <int D, int BN, int ST>
__device__ __forceinline__ char* k_slot(char* smem, int s) {
  return smem + s * (BN * D * 2);
}
template <int D, int BN, int ST>
__device__ __forceinline__ char* v_slot(char* smem, int s) {
  return smem + (ST + s) * (BN * D * 2);
}

// Wait until at most N of this wave's vector-memory operations are pending
// (copies complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads(): that fence
// makes the compiler wait for every outstanding vector-memory operation,
// including the LDS copies of later blocks, which would cap every ring at one
// block of copy latency. Callers wait for exactly the copies they need
// (wait_vmcnt) before it; this wave's LDS reads have returned when it passes.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane into LDS at lds_wave_base + 16 * lane through inline
// assembly, hidden from the compiler's wait tracking: its analysis does not
// treat the transposing LDS reads as disjoint from an in-flight copy and would
// drain every outstanding copy before them. Callers wait with wait_vmcnt; the
// memory clobber keeps LDS reads of the slot being overwritten in program
// order before the copy.
__device__ __forceinline__ void cs_dma(__amdgpu_buffer_rsrc_t r, int voff, char* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "s"(m0)
               : "m0", "memory");
}

// Chunk c of the key blocks [0, nblk): blocks [c*nblk/NC, (c+1)*nblk/NC),
// never empty when NC <= nblk.
__device__ __forceinline__ int chunk_begin(int c, int nblk, int nc) {
  return (int)(((long long)c * nblk) / nc);
}

constexpr int kDecodeMaxChunks = 2048;  // most key chunks a split-over-keys merge handles

}  // namespace

#endif  // ATTN_COMMON_H
