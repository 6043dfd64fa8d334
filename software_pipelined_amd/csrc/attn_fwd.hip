// Fused attention forward for MI355X (gfx950, CDNA4), behind the C ABI in
// include/attn.h.
//
// What is computed (PipeThreader, OSDI'25 summary page, "FlashAttention-3"
// paragraph and Fig 7; "PipeThreader and TileLang" page, section 4.1): per
// (batch, head) and per tile of query rows, stream K/V blocks (load_k,
// load_v), form S = Q K^T (mma_qk), keep an online softmax with a running
// row max and row sum (softmax), rescale the output accumulator (rescale),
// and accumulate O += P V (mma_pv); finally divide by the row sum and emit
// the row log-sum-exp.
//
// gfx950 mapping (not the pages' H100 design; their TMA producer warps and
// wgmma warp groups are prior art):
//   * a workgroup has NW wavefronts; each wave owns QT tiles of 32 query
//     rows end to end (BM = 32*QT*NW rows per workgroup);
//   * S is formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K (from LDS) is the A operand and Q^T (kept in registers for the whole
//     loop) the B operand, so each lane's accumulator column is one query and
//     row max / row sum reduce within the lane plus one lane^32 swap
//     (v_permlane32_swap); with QT = 2 every K fragment read from LDS feeds
//     two MFMAs;
//   * O^T += V^T P^T with the same instruction: P^T goes straight from the
//     S accumulators into the B operand (cvt to bf16, no LDS round trip),
//     V^T is read with the gfx950 transposing LDS read ds_read_b64_tr_b16;
//   * K/V blocks stream through an LDS ring filled with
//     buffer_load_dwordx4 ... lds (HBM -> LDS without VGPRs); the destination
//     layout is XOR-swizzled per row by choosing which global chunk each lane
//     fetches, so MFMA fragment reads are bank-conflict free;
//   * exp2 runs on v_exp_f32 with scale*log2(e) folded into one FMA;
//   * the O *= alpha rescale is skipped by a whole wave when none of its
//     rows raised its running max in the block (alpha == 1 exactly). The max
//     itself is tracked exactly, never lazily: a stale max makes the
//     dominant key's weight 2^delta instead of exactly 1, and its bf16
//     rounding then costs up to 2^-9 |v| on near-one-hot rows;
//   * workgroup ids are remapped so that consecutive query tiles of one head
//     run on one XCD (shared L2 for that head's K/V); causal grids start with
//     the heaviest tiles.
// Three schedules share the per-block step helpers (same arithmetic, bit for
// bit): "simple" (steps in program order), "pingpong" (two wave groups take
// turns on the matrix core) and "pipe" (each wave overlaps the softmax of
// block j with the QK^T MFMAs of block j+1).

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

// HBM -> LDS copies of BN-row blocks of one [N][D] matrix. Every wave moves
// LOADS x 1 KiB per block; lane l's 16 bytes land at dst + 16*l, so the
// swizzle is applied by choosing the source chunk. The source is a buffer
// resource over rows [row0, min(row0 + BN, N)): the hardware range check
// turns reads of rows past N into zeros (those keys are masked and their
// weights are exactly zero), so a copy needs no per-lane address arithmetic
// beyond its fixed lane offset.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ uint32_t block_lane_offset(int t, int wave, int lane) {
  using T = Tile<D, NW, BN>;
  const int p = (t * NW + wave) * 64 + lane;
  const int row = p / T::RC;
  const int pc = p % T::RC;
  const int c = pc ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
  return (uint32_t)(row * (D * 2) + c * 16);
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
template <int BN, int QT>
__device__ __forceinline__ void softmax_stats(const f32x16 (&s)[QT][BN / 32], float c_log2,
                                              float (&m_run)[QT], float (&alpha)[QT]) {
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
    const float m_new = fmaxf(m_run[qt], bmax * c_log2);
    alpha[qt] = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
    m_run[qt] = m_new;
  }
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
                                              float c_log2, float (&m_run)[QT], float (&l_run)[QT],
                                              float (&alpha)[QT]) {
  float ps[QT][4];
  softmax_stats<BN, QT>(s, c_log2, m_run, alpha);
  static_for<BN / 32>([&](auto KB) { softmax_exp<BN, QT, KB>(s, c_log2, m_run, ps); });
  softmax_pack<BN, QT>(s, pb);
  softmax_sum<QT>(l_run, alpha, ps);
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

// Load the wave's Q^T fragments (B operand of mma_qk): lane holds
// Q[q][kk*16 + h*8 .. +7] for its query q of each tile (rows past N clamped).
template <int D, int QT>
__device__ __forceinline__ void load_q(const uint16_t* Qh, int q0w, int N, int negate_q,
                                       bf16x8 (&qf)[QT][D / 16], int lane) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qrow = min(q0w + 32 * qt + (lane & 31), N - 1);
    const uint16_t* qp = Qh + (size_t)qrow * D + (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 raw = *(const u32x4*)(qp + kk * 16);
      if (negate_q) raw ^= 0x80008000u;  // exact sign flip of 8 bf16 values
      qf[qt][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
}

// Epilogue: O = O_acc / l and LSE = ln2 * (m + log2 l), stored for rows < N.
template <int D, int QT>
__device__ __forceinline__ void store_rows(float* O, float* LSE, size_t head, size_t bh, int N,
                                           int qi0, const f32x16 (&o)[QT][D / 32],
                                           const float (&m_run)[QT], const float (&l_run)[QT],
                                           int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = qi0 + 32 * qt;
    const float l_tot = swap32_sum(l_run[qt]);
    const float inv = 1.0f / l_tot;
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

// Everything a block step needs besides the per-block registers.
struct Ctx {
  const uint16_t* Kh;
  const uint16_t* Vh;
  size_t head;
  int bh;
  int N, nblk, kv_end_w, q0, q0w, qi0, wave, lane;
  float c_log2;
};

// Workgroup -> (batch*head, query tile) and the per-wave key range.
template <int D, int BM, int BN, int WROWS, bool CAUSAL>
__device__ __forceinline__ Ctx make_ctx(const uint16_t* K, const uint16_t* V, int N, int n_qtiles,
                                        float c_log2) {
  Ctx c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int tile;
  if (CAUSAL) {
    // Causal tiles differ in length. Heads are taken in groups, each inside
    // one XCD's contiguous range. Within a group the longest tiles of all its
    // heads come first (longest processing time first), so no long tile
    // starts at the end. A group's K/V stays within about twice an XCD's
    // 4 MB L2: 8 MiB / (K+V bytes per head) heads, at most BH/8. Measured
    // best on the causal N=2048 d=128, N=8192 d=64 and N=4096 d=256 shapes;
    // one head per group loses up to 18%, unbounded groups lose L2 reuse
    // (-24% at N=8192). The last group takes the remaining heads.
    const int BH = gridDim.x / n_qtiles;
    const int fit = (int)((8ll << 20) / (4ll * N * D));
    const int hpg = max(1, min(BH / 8, fit)), span = hpg * n_qtiles, ng = BH / hpg;
    const int g = L / span;
    const int h0 = min(g, ng) * hpg, hn = g < ng ? hpg : BH - ng * hpg;
    const int r = L - min(g, ng) * span;
    c.bh = h0 + r % hn;
    tile = n_qtiles - 1 - r / hn;
  } else {
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
  return c;
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
                                             f32x16 (&o)[QT][D / 32], float (&m_run)[QT],
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
  softmax_block<BN, QT>(s, pb, c.c_log2, m_run, l_run, alpha);
  rescale_block<D, QT>(o, alpha);
  pv_block<D, BN, QT>(v_slot<D, BN, ST>(smem, SLOT), off, pb, o);
  sched_mfma_with_reads<(BN / 16) * (D / 32), 2, QT, kPfPV>();
}

// OCC = workgroups per CU the register budget is sized for (waves per SIMD =
// NW * OCC / 4): with NW = 4 and OCC = 2 two independent workgroups share a
// CU, so the two waves on each SIMD are never held in step by one barrier.
template <int D, int NW, int BN, int QT, bool CAUSAL, int ST, int OCC>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_simple(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int negate_q) {
  using T = Tile<D, NW, BN, QT, ST>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const Ctx c = make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2);

  // Q first, then blocks 0 .. ST-2 (so the in-loop waits count block copies only)
  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, negate_q, qf, c.lane);
  if constexpr (NW * OCC <= 4) park_in_agprs<QT, D / 16>(qf);
#pragma unroll
  for (int b = 0; b < ST - 1; ++b)
    if (b < c.nblk) {
      issue_block_load<D, NW, BN, false>(c.Kh, b * BN, N, k_slot<D, BN, ST>(smem, b), c.wave, c.lane);
      issue_block_load<D, NW, BN, true>(c.Vh, b * BN, N, v_slot<D, BN, ST>(smem, b), c.wave, c.lane);
    }
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }
  for (int j = 0; j < c.nblk; j += ST) {
    simple_block<D, NW, BN, QT, CAUSAL, ST, 0>(c, smem, j, off, qf, o, m_run, l_run);
    if (j + 1 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 1 % ST>(c, smem, j + 1, off, qf, o, m_run, l_run);
    if (ST > 2 && j + 2 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 2 % ST>(c, smem, j + 2, off, qf, o, m_run, l_run);
    if (ST > 3 && j + 3 < c.nblk) simple_block<D, NW, BN, QT, CAUSAL, ST, 3 % ST>(c, smem, j + 3, off, qf, o, m_run, l_run);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, l_run, c.lane);
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
                                                f32x16 (&o)[QT][D / 32], float (&m_run)[QT],
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
  softmax_stats<BN, QT>(s_cur, c.c_log2, m_run, alpha);
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
                                                   float (&m_run)[QT], float (&l_run)[QT]) {
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
    softmax_stats<BN, QT>(s_cur, c.c_log2, m_run, alpha);
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
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_pipelined(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int negate_q) {
  static_assert(ST % 2 == 0, "the block loop is unrolled by ST and S alternates by parity");
  using T = Tile<D, NW, BN, QT, ST>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const Ctx c = make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2);

  // prologue: Q; K_0 .. K_{ST-1} and V_0 .. V_{ST-3} in flight; S_0 = Q K_0^T
  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, negate_q, qf, c.lane);
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
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
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
  pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, 0>(c, smem, 0, off, qf, sa, sb, pb, o, m_run, l_run);
  int j = 1;
  for (; j + ST - 1 < jf; j += ST) {
    static_for<ST>([&](auto I) {
      constexpr int slot = (1 + I) % ST;
      if constexpr ((1 + I) % 2)
        pipe_block_fast<D, NW, BN, QT, ST, slot>(c, smem, j + I, off, qf, sb, sa, pb, o, m_run, l_run);
      else
        pipe_block_fast<D, NW, BN, QT, ST, slot>(c, smem, j + I, off, qf, sa, sb, pb, o, m_run, l_run);
    });
  }
  for (; j < n; j += ST) {
    static_for<ST>([&](auto I) {
      constexpr int slot = (1 + I) % ST;
      if (j + I < n) {
        if constexpr ((1 + I) % 2)
          pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, slot>(c, smem, j + I, off, qf, sb, sa, pb, o, m_run, l_run);
        else
          pipe_block_generic<D, NW, BN, QT, CAUSAL, ST, slot>(c, smem, j + I, off, qf, sa, sb, pb, o, m_run, l_run);
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
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, l_run, c.lane);
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
                                                   f32x16 (&o)[QT][D / 32], float (&m_run)[QT],
                                                   float (&l_run)[QT], CopyFn&& copy) {
  constexpr int NB = BN / 32;
  __builtin_amdgcn_s_setprio(0);
  if (j < c.nblk && j * BN < c.kv_end_w) {
    const int kv0 = j * BN;
#pragma unroll
    for (int ci = 0; ci < NCOPY / 2; ++ci) copy(ci);
    if (block_needs_mask<BN, CAUSAL>(c, kv0)) mask_block<BN, QT, CAUSAL>(s, kv0, c.qi0, c.N, c.lane);
    float alpha[QT], ps[QT][4];
    softmax_stats<BN, QT>(s, c.c_log2, m_run, alpha);
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

template <int D, int NW, int BN, int QT, bool CAUSAL, int OCC>
__global__ __launch_bounds__(NW * 64, (NW * OCC + 3) / 4) void attn_fwd_pingpong(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int negate_q) {
  using T = Tile<D, NW, BN, QT, 2>;
  static_assert(NW % 2 == 0, "two wave groups");
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const Ctx c = make_ctx<D, T::BM, BN, 32 * QT, CAUSAL>(K, V, N, n_qtiles, c_log2);

  bf16x8 qf[QT][D / 16];
  load_q<D, QT>(Q + c.head, c.q0w, N, negate_q, qf, c.lane);
  issue_block_load<D, NW, BN, false>(c.Kh, 0, N, k_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  issue_block_load<D, NW, BN, true>(c.Vh, 0, N, v_slot<D, BN, 2>(smem, 0), c.wave, c.lane);
  if (c.nblk > 1)
    issue_block_load<D, NW, BN, false>(c.Kh, BN, N, k_slot<D, BN, 2>(smem, 1), c.wave, c.lane);
  const LdsOffsets<D> off(c.lane);
  f32x16 o[QT][D / 32];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qt][t] = f32x16{};
    m_run[qt] = -INFINITY;
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
      block_barrier();
      pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j, s, pb, o, m_run, l_run, no_copy);
      {
        auto copy = pingpong_odd_barrier<D, NW, BN, 0>(c, smem, j);
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, j, off, qf, s, pb, o, 1, copy);
      }
      if (j + 1 < n) {  // block j+1 (odd): slots swap
        block_barrier();
        pingpong_valu_turn<D, BN, QT, CAUSAL, 0>(c, j + 1, s, pb, o, m_run, l_run, no_copy);
        auto copy = pingpong_odd_barrier<D, NW, BN, 1>(c, smem, j + 1);
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, j + 1, off, qf, s, pb, o, 1, copy);
      }
    }
    block_barrier();  // t = 2n: group B's last mma_pv
  } else {
    for (int j = 0; j < n; j += 2) {
      // block j (even): [t=2j] pv(j-1) from V slot 1, qk(j) from K slot 0 | [t=2j+1] softmax
      block_barrier();
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, j - 1, off, qf, s, pb, o, 0, no_copy);
      {
        auto copy = pingpong_odd_barrier<D, NW, BN, 0>(c, smem, j);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j, s, pb, o, m_run, l_run, copy);
      }
      if (j + 1 < n) {
        block_barrier();
        pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, j, off, qf, s, pb, o, 0, no_copy);
        auto copy = pingpong_odd_barrier<D, NW, BN, 1>(c, smem, j + 1);
        pingpong_valu_turn<D, BN, QT, CAUSAL, 2 * LD>(c, j + 1, s, pb, o, m_run, l_run, copy);
      }
    }
    block_barrier();  // t = 2n: mma_pv of the last block, from V slot (n-1) & 1
    if (n & 1)
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 0, 1>(c, smem, n - 1, off, qf, s, pb, o, 0, no_copy);
    else
      pingpong_mfma_turn<D, NW, BN, QT, CAUSAL, 1, 0>(c, smem, n - 1, off, qf, s, pb, o, 0, no_copy);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  store_rows<D, QT>(O, LSE, c.head, c.bh, N, c.qi0, o, m_run, l_run, c.lane);
}

// ---------------------------------------------------------------- split-KV decoding
// Decoding step (split-KV / FlashDecoding in the pages' microbenchmarks):
// Nq query rows per (batch, head) against a cache of Nkv keys, every query
// seeing every key. Few query rows leave the matrix cores nearly idle, so the
// work is split over the keys instead: the key blocks of one (batch, head,
// 32-row query tile) are dealt to NC chunks, each processed by one wave with
// its own online softmax (the same per-block steps as the forward kernels) and
// written as a normalised partial (O_c, LSE_c) to the caller's workspace. A
// second kernel merges the chunks of each row: LSE = ln sum_c exp(LSE_c),
// O = sum_c exp(LSE_c - LSE) O_c. The pass is HBM-bound (K and V are read
// once), so each wave streams its own chunk through a private LDS ring and
// never waits on the other waves of its workgroup.

// HBM -> LDS copy issued through inline assembly. The compiler's wait
// analysis does not treat the transposing LDS reads as disjoint from an
// in-flight copy, and would wait for every outstanding copy before each V
// read (no overlap of the next block's copy with this block's math); hidden
// from it, the copies are waited for explicitly (wait_vmcnt) instead. The
// memory clobber keeps LDS reads of the slot being overwritten in program
// order before the copy.
template <int D, int BN, bool IS_V>
__device__ __forceinline__ void issue_copy_wave(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                                int lane, int t) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc<D, BN>(src, row0, N);
  const int off = (int)block_lane_offset<D, 1, BN, IS_V>(t, 0, lane);
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)(dst + t * 64 * 16);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "s"(m0)
               : "m0", "memory");
}

template <int D, int BN>
__device__ __forceinline__ void copy_block_wave(const uint16_t* Kh, const uint16_t* Vh, int row0, int N,
                                                char* ks, char* vs, int lane) {
  constexpr int LD = Tile<D, 1, BN>::LOADS;
#pragma unroll
  for (int t = 0; t < LD; ++t) {
    issue_copy_wave<D, BN, false>(Kh, row0, N, ks, lane, t);
    issue_copy_wave<D, BN, true>(Vh, row0, N, vs, lane, t);
  }
}

// Chunk c of the key blocks [0, nblk): blocks [c*nblk/NC, (c+1)*nblk/NC),
// never empty when NC <= nblk.
__device__ __forceinline__ int chunk_begin(int c, int nblk, int nc) {
  return (int)(((long long)c * nblk) / nc);
}

// Grid: (B*H*n_qt) x (NC / NW) workgroups of NW waves; wave w of workgroup
// (x, y) takes chunk y*NW + w of query tile x % n_qt of head x / n_qt.
template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void attn_decode_partial(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int BH, int Nq, int Nkv, int n_qt, int nc,
    float c_log2, int negate_q) {
  constexpr int ST = 2;
  constexpr int MAT = BN * D * 2;
  constexpr int PER_BLOCK = 2 * Tile<D, 1, BN>::LOADS;
  __shared__ __attribute__((aligned(1024))) char smem[NW * ST * 2 * MAT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x / n_qt, qt0 = (blockIdx.x % n_qt) * 32;
  const int c = blockIdx.y * NW + wave;
  const int nblk = (Nkv + BN - 1) / BN;
  const int b0 = chunk_begin(c, nblk, nc), b1 = chunk_begin(c + 1, nblk, nc);
  const uint16_t* Kh = K + (size_t)bh * Nkv * D;
  const uint16_t* Vh = V + (size_t)bh * Nkv * D;
  char* ring = smem + wave * (ST * 2 * MAT);
  auto ks = [ring](int s) { return ring + s * MAT; };
  auto vs = [ring](int s) { return ring + (ST + s) * MAT; };

  bf16x8 qf[1][D / 16];
  load_q<D, 1>(Q + (size_t)bh * Nq * D, qt0, Nq, negate_q, qf, lane);
  if constexpr (NW <= 4) park_in_agprs<1, D / 16>(qf);
  const LdsOffsets<D> off(lane);
  f32x16 o[1][D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[0][t] = f32x16{};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};

  if (b0 == b1) {  // an empty chunk (fewer key blocks than chunks): weight zero in the merge
    const int qi = qt0 + (lane & 31);
    if (qi < Nq) {
      float* orow = ws_o + ((size_t)c * BH * Nq + (size_t)bh * Nq + qi) * D;
      for (int e = (lane >> 5); e < D; e += 2) orow[e] = 0.f;
      if (lane < 32) ws_lse[(size_t)c * BH * Nq + (size_t)bh * Nq + qi] = -INFINITY;
    }
    return;
  }
  copy_block_wave<D, BN>(Kh, Vh, b0 * BN, Nkv, ks(0), vs(0), lane);
  for (int j = b0; j < b1; ++j) {
    const int slot = (j - b0) & 1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the slot about to be refilled are done
    if (j + 1 < b1) {
      copy_block_wave<D, BN>(Kh, Vh, (j + 1) * BN, Nkv, ks(slot ^ 1), vs(slot ^ 1), lane);
      wait_vmcnt<PER_BLOCK>();  // block j has landed, block j+1 may stay in flight
    } else {
      wait_vmcnt<0>();
    }
    const char* kslot = ks(slot);
    const char* vslot = vs(slot);
    f32x16 s[1][BN / 32];
    qk_block<D, BN, 1>(kslot, off, qf, s);
    sched_mfma_with_reads<(D / 16) * (BN / 32), 1, 1, kPfQK>();
    const int kv0 = j * BN;
    if (kv0 + BN > Nkv) mask_block<BN, 1, false>(s, kv0, 0, Nkv, lane);
    bf16x8 pb[1][BN / 16];
    float alpha[1];
    softmax_block<BN, 1>(s, pb, c_log2, m_run, l_run, alpha);
    rescale_block<D, 1>(o, alpha);
    pv_block<D, BN, 1>(vslot, off, pb, o);
    sched_mfma_with_reads<(BN / 16) * (D / 32), 2, 1, kPfPV>();
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the wave
  store_rows<D, 1>(ws_o + (size_t)c * BH * Nq * D, ws_lse + (size_t)c * BH * Nq, (size_t)bh * Nq * D,
                   (size_t)bh, Nq, qt0 + (lane & 31), o, m_run, l_run, lane);
}

// One workgroup per query row merges the row's NC chunk partials: the chunk
// weights exp(LSE_c - max) are formed once in LDS, while each thread already
// holds its first partials in registers; each thread sums one output
// dimension over a slice of the chunks (coalesced across threads) and the
// slices are added in LDS.
constexpr int kDecodeMaxChunks = 2048;  // the planner never makes more

template <int D>
__global__ __launch_bounds__(256, 1) void attn_decode_combine(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_lse,
                                                             float* __restrict__ O, float* __restrict__ LSE,
                                                             int rows, int nc) {
  constexpr int G = 256 / D;  // chunk slices
  __shared__ float w_sh[kDecodeMaxChunks];
  __shared__ float red[256];
  constexpr int PF = 32;      // partials per thread loaded before the weights are known
  const int tid = threadIdx.x, row = blockIdx.x;
  const int dim = tid % D, g = tid / D;
  float pre[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int c = g + i * G;
    pre[i] = c < nc ? ws_o[((size_t)c * rows + row) * D + dim] : 0.f;
  }
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += 256) {
    const float l = ws_lse[(size_t)c * rows + row];
    w_sh[c] = l;
    mx = fmaxf(mx, l);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float ws = 0.f;
  for (int c = tid; c < nc; c += 256) {
    const float w = __builtin_amdgcn_exp2f((w_sh[c] - mx) * kLog2e);  // 0 for an empty chunk
    w_sh[c] = w;
    ws += w;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) ws += __shfl_xor(ws, sh);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = ws;
  __syncthreads();  // also publishes every weight in w_sh
  const float wsum = (red[4] + red[5]) + (red[6] + red[7]);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int c = g + i * G;
    if (c < nc) acc += w_sh[c] * pre[i];
  }
  int c = g + PF * G;
  for (; c + 3 * G < nc; c += 4 * G) {
    const float* src = ws_o + ((size_t)c * rows + row) * D + dim;
    const size_t st = (size_t)G * rows * D;
    acc += w_sh[c] * src[0] + w_sh[c + G] * src[st] + w_sh[c + 2 * G] * src[2 * st] +
           w_sh[c + 3 * G] * src[3 * st];
  }
  for (; c < nc; c += G) acc += w_sh[c] * ws_o[((size_t)c * rows + row) * D + dim];
  __syncthreads();  // every thread has read red[4..7]
  red[tid] = acc;
  __syncthreads();
  if (tid < D) {
    float o = red[tid];
#pragma unroll
    for (int k = 1; k < G; ++k) o += red[tid + k * D];
    O[(size_t)row * D + tid] = o / wsum;
  }
  if (tid == 0) LSE[row] = mx + kLn2 * __builtin_amdgcn_logf(wsum);
}

// ---------------------------------------------------------------- backward
// The gradient of the forward (the attention backward that the Twill
// write-up schedules in its section 3.2; the pages do not restate it, so it
// is the derivative of the forward's definition). With dO the gradient of O:
//   D_i = sum_c dO_ic O_ic,  P_ij = exp(s_ij - LSE_i),  dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,
//   dQ_i = scale sum_j dS_ij k_j.
// Three kernels: attn_bwd_prep (D and log2-scaled LSE, per 32-row query
// block), attn_bwd_dkdv (a workgroup owns key tiles and streams every query
// block that sees them: dK and dV never leave registers) and attn_bwd_dq (a
// workgroup owns query tiles and streams the key blocks, recomputing S and dP:
// dQ needs dS with keys as the contraction, the transpose of what the
// key-owning kernel holds, and recomputation avoids atomics, so results are
// deterministic).
//
// Layout tricks shared by both main kernels: a [rows][d] block image in LDS
// (K-style XOR swizzle) serves both as row-fragment A operand
// (ds_read_b128) and, through ds_read_b64_tr_b16, as the transposed A
// operand; an MFMA accumulator tile converted to bf16 is the B operand of the
// next product without an LDS round trip.

constexpr int kBwdRows = 32;               // query rows per statistics block
constexpr int kBwdStatBytes = 2 * kBwdRows * 4;  // log2e*LSE then D, fp32

// Compact fragment offsets into a K-swizzled [rows][D] image, one or two
// registers per lane instead of one per fragment: the swizzle only permutes
// 16-byte chunks within a row, so every fragment's offset is one lane base
// XOR a compile-time constant (the row part and the chunk part occupy
// disjoint bits).
//   row fragment kk (A operand, ds_read_b128): row lq, chunk 2kk + h
//       = kbase ^ (32 kk);
//   transposed read (t, r) (ds_read_b64_tr_b16, as LdsOffsets::v): rows
//       r0 + 8r carry different swizzles, so two bases; dims tile t
//       = tbase[r] ^ (64 t); adding 16p rows leaves the swizzle unchanged.
template <int D>
struct BwdOffsets {
  int kbase, tbase0, tbase1;
  __device__ __forceinline__ explicit BwdOffsets(int lane) {
    const int h = lane >> 5, lq = lane & 31, ci = lane & 15, g2 = (lane >> 4) & 1;
    kbase = lq * (D * 2) + ((h ^ swz_k<D>(lq)) << 4);
    const int r0 = 4 * h + (ci >> 2), c1 = 2 * g2 + ((ci & 3) >> 1);
    tbase0 = r0 * (D * 2) + ((c1 ^ swz_k<D>(r0)) << 4) + 8 * (ci & 1);
    tbase1 = r0 * (D * 2) + ((c1 ^ swz_k<D>(r0 + 8)) << 4) + 8 * (ci & 1);
  }
  __device__ __forceinline__ int k(int kk) const { return kbase ^ (32 * kk); }
};

// A operand of X^T[dim tile t][rows 16p .. 16p+15] from a K-swizzled image.
template <int D>
__device__ __forceinline__ bf16x8 read_tr_k(const char* img, const BwdOffsets<D>& bo, int t, int p) {
  const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(img + (bo.tbase0 ^ (64 * t)) + (p * 16) * (D * 2)));
  const i16x4 a1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(img + (bo.tbase1 ^ (64 * t)) + (p * 16 + 8) * (D * 2)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup-shared HBM -> LDS copy t of a BN-row block (same placement as
// issue_copy, K swizzle), in inline assembly so that the compiler's
// conservative wait before transposed LDS reads does not drain the copies of
// the next block; callers wait with wait_vmcnt.
template <int D, int NW, int BN>
__device__ __forceinline__ void issue_copy_asm(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                               int wave, int lane, int t) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc<D, BN>(src, row0, N);
  const int off = (int)block_lane_offset<D, NW, BN, false>(t, wave, lane);
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)(dst + (t * NW + wave) * 64 * 16);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "s"(m0)
               : "m0", "memory");
}

// One 256-byte statistics block into a wave's own 1 KiB LDS slot (lanes past
// the block read zeros).
__device__ __forceinline__ void issue_stat_copy(const float* src, char* dst, int lane) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, kBwdStatBytes, kRsrcWord3);
  const int off = lane * 16;
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)dst;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "s"(m0)
               : "m0", "memory");
}

// stats[bh][blk] = { log2e * LSE of the block's 32 rows, D of those rows };
// rows past N get +inf (so exp2(s*c - inf) = 0) and 0. One workgroup per
// block: 8 threads per row, each summing d/8 products.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep(const float* __restrict__ O, const uint16_t* __restrict__ dO,
                                                    const float* __restrict__ LSE, float* __restrict__ stats,
                                                    int N, int nqb) {
  const int blk = blockIdx.x % nqb, bh = blockIdx.x / nqb;
  const int tid = threadIdx.x, row = tid >> 3, part = tid & 7;
  const int i = blk * kBwdRows + row;
  float acc = 0.f;
  if (i < N) {
    const size_t base = ((size_t)bh * N + i) * D;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const int e = c * 64 + part * 8;
      const u32x4 g = *(const u32x4*)(dO + base + e);
      const f32x4 o0 = *(const f32x4*)(O + base + e), o1 = *(const f32x4*)(O + base + e + 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += __uint_as_float(g[w] << 16) * (w < 2 ? o0[2 * w] : o1[2 * w - 4]);
        acc += __uint_as_float(g[w] & 0xFFFF0000u) * (w < 2 ? o0[2 * w + 1] : o1[2 * w - 3]);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (part == 0) {
    float* st = stats + ((size_t)bh * nqb + blk) * (2 * kBwdRows);
    st[row] = i < N ? LSE[(size_t)bh * N + i] * kLog2e : INFINITY;
    st[kBwdRows + row] = i < N ? acc : 0.f;
  }
}

// dK, dV. Workgroup = NW waves, wave w owns keys k0 + 32w .. +31 (K and V
// rows as B-operand registers). Query blocks of 32 rows (Q, dO, statistics)
// stream through a two-stage LDS ring. Per block and wave:
//   S = Q K^T, dP = dO V^T          (A = Q / dO row fragments, B = K / V)
//   P = exp2(c*S - log2e*LSE), dS = P (dP - D)   (accumulator layout: query rows)
//   dV^T += dO^T P, dK^T += Q^T dS  (A = transposed reads, B = P / dS in bf16)
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ stats, float* __restrict__ dK,
    float* __restrict__ dV, int N, int n_ktiles, float c_log2, int negate, float scale) {
  constexpr int BQ = kBwdRows;
  constexpr int MAT = BQ * D * 2;
  constexpr int LD = Tile<D, NW, BQ>::LOADS;
  constexpr int STAT = 1024;
  constexpr int STAGE = 2 * MAT + NW * STAT;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_ktiles, kt = L % n_ktiles;
  const int k0 = kt * 32 * NW, k0w = k0 + 32 * wave;
  const size_t head = (size_t)bh * N * D;
  const int nqb = (N + BQ - 1) / BQ;
  const float* st_head = stats + (size_t)bh * nqb * (2 * BQ);

  bf16x8 kf[1][D / 16], vf[1][D / 16];
  load_q<D, 1>(K + head, k0w, N, negate, kf, lane);  // scale < 0: S from -K, c = |scale| log2e
  load_q<D, 1>(V + head, k0w, N, 0, vf, lane);
  const BwdOffsets<D> bo(lane);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dk[t] = dv[t] = f32x16{};

  auto copy_stage = [&](int jb, int slot) {
    char* base = smem + slot * STAGE;
#pragma unroll
    for (int t = 0; t < LD; ++t) {
      issue_copy_asm<D, NW, BQ>(Q + head, jb * BQ, N, base, wave, lane, t);
      issue_copy_asm<D, NW, BQ>(dO + head, jb * BQ, N, base + MAT, wave, lane, t);
    }
    issue_stat_copy(st_head + (size_t)jb * (2 * BQ), base + 2 * MAT + wave * STAT, lane);
  };

  const int jb0 = CAUSAL ? min(k0 / BQ, nqb) : 0;  // earlier query blocks see none of these keys
  if (jb0 < nqb) copy_stage(jb0, 0);
  const int key = k0w + (lane & 31);
  for (int jb = jb0; jb < nqb; ++jb) {
    const int slot = (jb - jb0) & 1;
    wait_vmcnt<0>();
    block_barrier();
    if (jb + 1 < nqb) copy_stage(jb + 1, slot ^ 1);
    const char* Qs = smem + slot * STAGE;
    const char* dOs = Qs + MAT;
    const char* Ss = Qs + 2 * MAT + wave * STAT;
    const int q0 = jb * BQ;
    if (CAUSAL && q0 + BQ - 1 < k0w) continue;  // wave-uniform: every query precedes every key of this wave
    // fragments are read right before the MFMA that consumes them: with two
    // waves per SIMD the K/V operands and dK/dV accumulators leave little room
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(LDS_AS const bf16x8*)(Qs + bo.k(kk)), kf[0][kk], s, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(LDS_AS const bf16x8*)(dOs + bo.k(kk)), vf[0][kk], dp, 0, 0, 0);
    const bool diag = CAUSAL && q0 < k0w + 31;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2 = *(LDS_AS const f32x4*)(Ss + (8 * g + 4 * h) * 4);
      const f32x4 dd = *(LDS_AS const f32x4*)(Ss + BQ * 4 + (8 * g + 4 * h) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2[i]));
        if (diag) {
          const int qi = q0 + 8 * g + 4 * h + i;
          p = key > qi ? 0.f : p;
        }
        s[r] = p;
        dp[r] = p * (dp[r] - dd[i]);
      }
    }
    bf16x8 pb[1][2], dsb[1][2];
    softmax_pack<32, 1>(*(const f32x16(*)[1][1])&s, pb);
    softmax_pack<32, 1>(*(const f32x16(*)[1][1])&dp, dsb);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const bf16x8 ado = read_tr_k<D>(dOs, bo, t, p);
        const bf16x8 aq = read_tr_k<D>(Qs, bo, t, p);
        dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ado, pb[0][p], dv[t], 0, 0, 0);
        dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsb[0][p], dk[t], 0, 0, 0);
      }
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  if (key < N) {
    float* krow = dK + head + (size_t)key * D;
    float* vrow = dV + head + (size_t)key * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = t * 32 + g * 8 + h * 4;
        *(f32x4*)(krow + e) = f32x4{dk[t][4 * g] * scale, dk[t][4 * g + 1] * scale, dk[t][4 * g + 2] * scale,
                                    dk[t][4 * g + 3] * scale};
        *(f32x4*)(vrow + e) = f32x4{dv[t][4 * g], dv[t][4 * g + 1], dv[t][4 * g + 2], dv[t][4 * g + 3]};
      }
  }
}

// dQ. Workgroup = NW waves, wave w owns queries q0 + 32w .. +31 (Q and dO as
// B-operand registers, its LSE and D in one register each); key blocks of BN
// rows (K, V) stream through a two-stage LDS ring. Per block and wave:
//   S^T = K Q^T, dP^T = V dO^T      (the forward's mma_qk, twice)
//   dS^T = exp2(c*S^T - log2e*LSE) (dP^T - D)   (masked keys: 0)
//   dQ^T += K^T dS^T                (A = transposed reads of the K image)
template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ stats, float* __restrict__ dQ, int N,
    int n_qtiles, float c_log2, int negate, float scale) {
  constexpr int MAT = BN * D * 2;
  constexpr int LD = Tile<D, NW, BN>::LOADS;
  constexpr int STAGE = 2 * MAT;
  constexpr int BMQ = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qtiles;
  const int qt = CAUSAL ? n_qtiles - 1 - L % n_qtiles : L % n_qtiles;  // causal: longest first
  const int q0 = qt * BMQ, q0w = q0 + 32 * wave, qi = q0w + (lane & 31);
  const size_t head = (size_t)bh * N * D;
  const int nqb = (N + kBwdRows - 1) / kBwdRows;

  bf16x8 qf[1][D / 16], gf[1][D / 16];
  load_q<D, 1>(Q + head, q0w, N, negate, qf, lane);  // scale < 0: S from -Q, c = |scale| log2e
  load_q<D, 1>(dO + head, q0w, N, 0, gf, lane);
  const int qs = min(qi, nqb * kBwdRows - 1);  // rows past N: padded statistics (+inf, 0)
  const float* st = stats + ((size_t)bh * nqb + qs / kBwdRows) * (2 * kBwdRows);
  const float l2 = st[qs % kBwdRows], dd = st[kBwdRows + qs % kBwdRows];
  const LdsOffsets<D> off(lane);
  const BwdOffsets<D> bo(lane);
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dq[t] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q0 + BMQ) : N;
  const int kv_end_w = CAUSAL ? min(N, q0w + 32) : N;
  const int nkb = (kv_end + BN - 1) / BN;
  auto copy_stage = [&](int jb, int slot) {
    char* base = smem + slot * STAGE;
#pragma unroll
    for (int t = 0; t < LD; ++t) {
      issue_copy_asm<D, NW, BN>(K + head, jb * BN, N, base, wave, lane, t);
      issue_copy_asm<D, NW, BN>(V + head, jb * BN, N, base + MAT, wave, lane, t);
    }
  };
  copy_stage(0, 0);
  for (int jb = 0; jb < nkb; ++jb) {
    const int slot = jb & 1;
    wait_vmcnt<0>();
    block_barrier();
    if (jb + 1 < nkb) copy_stage(jb + 1, slot ^ 1);
    const int kv0 = jb * BN;
    if (kv0 >= kv_end_w) continue;  // wave-uniform: every key of the block follows every query of this wave
    const char* Ks = smem + slot * STAGE;
    const char* Vs = Ks + MAT;
    f32x16 s[1][BN / 32], dp[1][BN / 32];
    qk_block<D, BN, 1>(Ks, off, qf, s);
    qk_block<D, BN, 1>(Vs, off, gf, dp);
    if (kv0 + BN > N || (CAUSAL && kv0 + BN - 1 > q0w)) mask_block<BN, 1, CAUSAL>(s, kv0, qi, N, lane);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][kb][r], c_log2, -l2));
        s[0][kb][r] = p * (dp[0][kb][r] - dd);
      }
    bf16x8 dsb[1][BN / 16];
    softmax_pack<BN, 1>(s, dsb);
#pragma unroll
    for (int p = 0; p < BN / 16; ++p)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr_k<D>(Ks, bo, t, p), dsb[0][p], dq[t], 0, 0, 0);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  if (qi < N) {
    float* qrow = dQ + head + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(qrow + t * 32 + g * 8 + h * 4) = f32x4{dq[t][4 * g] * scale, dq[t][4 * g + 1] * scale,
                                                        dq[t][4 * g + 2] * scale, dq[t][4 * g + 3] * scale};
  }
}

// ---------------------------------------------------------------- Mamba2 ChunkScan
// PipeThreader summary page, "Running example: Mamba2" and Fig 6(a): inside
// each chunk of L steps, cb is scaled by the exponential decay built from dA
// and by dt, and its product with x accumulates into the output:
//   out[b][s][h][:] = sum_{k <= m} cb[b][c][m][k] exp(dAc[m] - dAc[k]) dt[k] x[b][cL+k][h][:]
// (m = s - cL, dAc = the running sum of dA within the chunk). The same MFMA
// mapping as the forward's mma_pv: out^T[p][m] += x^T[p][k] A^T[k][m] with
// A[m][k] = cb[m][k] exp(dAc[m] - dAc[k]) dt[k] formed in registers straight
// into the B-operand layout (so A never exists in memory) and x^T read from
// an LDS image of the 32-step block with the transposing LDS read. One
// workgroup per (b, chunk, h): 4 waves, wave w owns chunk rows 64w .. 64w+63;
// every input of a 32-step block (x, the cb columns, dt, dA_cumsum) streams
// through a two-slot LDS ring, so the next block's loads are in flight while
// this one is computed. Workgroup ids run over heads fastest, so the heads
// sharing one cb chunk run together.
constexpr int kCsP = 64;   // channels per head
constexpr int kCsBK = 32;  // steps per block
// One ring slot: the x block (32 x 64 bf16, V layout), the cb columns of the
// block for all 256 possible rows (64 bytes per row, 16-byte chunks XORed
// with (row >> 1) & 3), then dt and dA_cumsum of the block's 32 steps (one
// 1 KiB copy each, only the first 128 bytes used).
constexpr int kCsX = kCsBK * kCsP * 2;
template <int RW>
struct CsSlot {
  static constexpr int CB = RW * kCsBK * 2;    // cb columns of the block for the workgroup's RW rows
  static constexpr int BYTES = kCsX + CB + 2 * 1024;
};

// 16 bytes per lane into LDS at lds_wave_base + 16 * lane, hidden from the
// compiler's wait tracking (callers wait with wait_vmcnt).
__device__ __forceinline__ void cs_dma(__amdgpu_buffer_rsrc_t r, int voff, char* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "s"(m0)
               : "m0", "memory");
}

// All copies of block j (steps k0 = 32j ..): x rows (rows past the chunk
// read zeros), the cb columns k0 .. k0+31 of the workgroup's rows
// [max(k0, r0), min(L, r0 + RW)) (earlier rows never see the block), dt and
// dA_cumsum.
template <int NW, int RW>
__device__ __forceinline__ void cs_copy_block(const uint16_t* xh, const uint16_t* cbc, const float* dtc,
                                              const float* dac, int j, int Lc, int L, int r0, int row_stride,
                                              char* slot, int wave, int lane) {
  const int k0 = j * kCsBK;
  {  // x: one 1 KiB copy per wave (8 rows)
    const int pidx = wave * 64 + lane;
    const int row = pidx >> 3, pc = pidx & 7;
    const int rows_valid = min(kCsBK, Lc - k0);
    const int bytes = __builtin_amdgcn_readfirstlane((rows_valid - 1) * row_stride * 2 + kCsP * 2);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xh + (size_t)k0 * row_stride), (short)0, bytes, kRsrcWord3);
    cs_dma(r, row * row_stride * 2 + ((pc ^ swz_v<kCsP>(row)) << 4), slot + wave * 1024);
  }
  {  // cb: rows of 64 bytes, 16 per 1 KiB copy, dealt over the waves
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)cbc, (short)0, L * L * 2, kRsrcWord3);
    const int first = max(k0, r0), n = (min(L, r0 + RW) - first) / 16;
    for (int t = wave; t < n; t += NW) {
      const int pidx = t * 64 + lane;
      const int row = first + (pidx >> 2), pc = pidx & 3;
      const int c = pc ^ ((row >> 1) & 3);
      cs_dma(r, (row * L + k0) * 2 + (c << 4), slot + kCsX + (first - r0) * 64 + t * 1024);
    }
  }
  if (wave == 0) {  // dt and dA_cumsum of the block's 32 steps
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)(dtc + k0), (short)0, 128, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(dac + k0), (short)0, 128, kRsrcWord3);
    cs_dma(rd, lane * 16, slot + kCsX + CsSlot<RW>::CB);
    cs_dma(ra, lane * 16, slot + kCsX + CsSlot<RW>::CB + 1024);
  }
}

// QT 32-row tiles per wave: a workgroup covers RW = 32*QT*NW chunk rows
// starting at r0; a chunk takes ceil(L / RW) workgroups.
template <int NW, int QT>
__global__ __launch_bounds__(NW * 64) void chunk_scan_fwd(const uint16_t* __restrict__ X, const uint16_t* __restrict__ CB,
                                                         const float* __restrict__ DT, const float* __restrict__ DAC,
                                                         float* __restrict__ OUT, int S, int H, int L, int nc) {
  static_assert(NW == 4, "one 1 KiB copy per wave covers a 32 x 64 bf16 block");
  constexpr int RW = 32 * QT * NW;
  constexpr int SLOT = CsSlot<RW>::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT];
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nparts = (L + RW - 1) / RW;
  const int h = blockIdx.x % H, part = (blockIdx.x / H) % nparts, c = (blockIdx.x / (H * nparts)) % nc,
            b = blockIdx.x / (H * nparts * nc);
  const int c0 = c * L, Lc = min(L, S - c0), r0 = part * RW;
  if (r0 >= Lc) return;  // workgroup-uniform: this part of a short last chunk is empty
  const int nblk = (min(Lc, r0 + RW) + kCsBK - 1) / kCsBK;
  const int row_stride = H * kCsP;
  const uint16_t* xh = X + ((size_t)b * S + c0) * row_stride + (size_t)h * kCsP;
  const uint16_t* cbc = CB + ((size_t)b * nc + c) * L * L;
  const size_t sc = (((size_t)b * H + h) * nc + c) * L;
  const float* dtc = DT + sc;
  const float* dac = DAC + sc;
  const int mw = r0 + 32 * QT * wave;  // first chunk row of this wave

  float dam[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) dam[qt] = dac[min(mw + 32 * qt + (lane & 31), Lc - 1)];
  const LdsOffsets<kCsP> off(lane);
  f32x16 o[QT][kCsP / 32];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int t = 0; t < kCsP / 32; ++t) o[qt][t] = f32x16{};

  cs_copy_block<NW, RW>(xh, cbc, dtc, dac, 0, Lc, L, r0, row_stride, smem, wave, lane);
  for (int j = 0; j < nblk; ++j) {
    wait_vmcnt<0>();
    block_barrier();
    if (j + 1 < nblk)
      cs_copy_block<NW, RW>(xh, cbc, dtc, dac, j + 1, Lc, L, r0, row_stride, smem + ((j + 1) & 1) * SLOT, wave, lane);
    const int k0 = j * kCsBK;
    if (mw >= Lc || k0 > mw + 32 * QT - 1) continue;  // wave-uniform: no row of this wave sees the block
    const char* slot = smem + (j & 1) * SLOT;
    const char* cbs = slot + kCsX;
    const char* dts = cbs + CsSlot<RW>::CB;
    // dt and dA_cumsum of this lane's 16 steps: k0 + 16hf + 8e + 4hl + i
    f32x4 dtv[2][2], dav[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dtv[hf][e] = *(LDS_AS const f32x4*)(dts + (16 * hf + 8 * e + 4 * hl) * 4);
        dav[hf][e] = *(LDS_AS const f32x4*)(dts + 1024 + (16 * hf + 8 * e + 4 * hl) * 4);
      }
    bf16x8 pb[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int m = mw + 32 * qt + (lane & 31);
      const int sw = (m >> 1) & 3;
      const char* cbr = cbs + (m - r0) * 64 + 8 * hl;  // rows below k0 hold stale data; their terms are masked
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x2 raw = *(LDS_AS const u32x2*)(cbr + (((2 * hf + e) ^ sw) << 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = raw[i >> 1];
            const float cbv = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
            const int kk = k0 + 16 * hf + 8 * e + 4 * hl + i;
            const float decay = __builtin_amdgcn_exp2f((dam[qt] - dav[hf][e][i]) * kLog2e);
            a[4 * e + i] = kk <= m ? cbv * decay * dtv[hf][e][i] : 0.f;
          }
        }
        pb[qt][hf] = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                            (__bf16)a[4], (__bf16)a[5], (__bf16)a[6], (__bf16)a[7]};
      }
    }
    pv_block<kCsP, kCsBK, QT>(slot, off, pb, o);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int m = mw + 32 * qt + (lane & 31);
    if (m < Lc) {
      float* orow = OUT + (((size_t)b * S + c0 + m) * H + h) * kCsP;
#pragma unroll
      for (int t = 0; t < kCsP / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(orow + t * 32 + g * 8 + hl * 4) =
              f32x4{o[qt][t][4 * g], o[qt][t][4 * g + 1], o[qt][t][4 * g + 2], o[qt][t][4 * g + 3]};
    }
  }
}

// ---------------------------------------------------------------- MLA decoding
// Multi-head latent attention decoding in the absorbed form (the decoding
// operator the PipeThreader-and-TileLang page cites as a short TileLang
// program): all H query heads of a sequence attend to one shared cache of
// latent rows of Dk = 576 values (512 latent + 64 rotary); a row's first
// Dv = 512 values are its value. Split over key chunks like attn_fwd_decode
// (normalised partials merged by LSE weights), but a workgroup serves 64
// heads at once, so each cache block is read from HBM once per 64 heads:
// one LDS image of a 32-row block serves both S^T = K Q^T (row fragments) and
// O^T += V^T P^T (transposed reads of its first 512 columns). Four waves:
// wave = 2*tile + half takes the 32 heads of its tile and output dims
// [256*half, 256*half + 256); the two waves of a tile split the 576-wide
// contraction of S (288 each, their Q^T halves in AGPRs) and swap partial
// sums through LDS, so both hold the same S (a + b == b + a exactly).
constexpr int kMlaDk = 576, kMlaDv = 512, kMlaBN = 32;
constexpr int kMlaRow = kMlaDk * 2;             // bytes per cache row
constexpr int kMlaBlock = kMlaBN * kMlaRow;     // 36 KiB per 32-row block
constexpr int kMlaCopies = kMlaBlock / 1024;    // 1 KiB copies per block

// 16-byte chunk c of row `row` sits at chunk (c & ~7) | ((c ^ row) & 7): an
// XOR inside each group of eight chunks (a row has 72), an involution.
__device__ __forceinline__ int mla_phys(int c, int row) { return (c & ~7) | ((c ^ row) & 7); }

__device__ __forceinline__ void mla_copy_block(const uint16_t* kvb, int row0, int N, char* dst, int wave, int lane) {
  const int rows = __builtin_amdgcn_readfirstlane(min(N - row0, kMlaBN));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(kvb + (size_t)row0 * kMlaDk), (short)0,
                                                                     rows * kMlaRow, kRsrcWord3);
#pragma unroll
  for (int t = 0; t < kMlaCopies / 4; ++t) {
    const int pidx = (t * 4 + wave) * 64 + lane;
    const int row = pidx / 72, pc = pidx % 72;
    cs_dma(r, row * kMlaRow + (mla_phys(pc, row) << 4), dst + (t * 4 + wave) * 1024);
  }
}

// Grid: (B * H/64) x NC. Chunk c of the key blocks as chunk_begin.
constexpr int kMlaHalfK = kMlaDk / 32;  // 16-wide contraction steps per wave (18)
constexpr int kMlaST = 3;                 // ring slots: two blocks in flight behind the one in use
constexpr int kMlaXchg = 4 * 64 * 64;     // partial-S exchange: 64 bytes per lane per wave

__global__ __launch_bounds__(256, 1) void mla_decode_partial(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ KV,
                                                            float* __restrict__ ws_o, float* __restrict__ ws_lse,
                                                            int N, int H, int nc, float c_log2, int negate_q) {
  static_assert(kMlaCopies % 4 == 0, "copies split evenly over four waves");
  __shared__ __attribute__((aligned(1024))) char smem[kMlaST * kMlaBlock + kMlaXchg];
  const int lane = threadIdx.x & 63, hl = lane >> 5, lq = lane & 31, ci = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = wave >> 1, half = wave & 1;
  const int hg = H / 64;
  const int b = blockIdx.x / hg, h0 = (blockIdx.x % hg) * 64 + 32 * tile;
  const int c = blockIdx.y;
  const int nblk = (N + kMlaBN - 1) / kMlaBN;
  const int b0 = chunk_begin(c, nblk, nc), b1 = chunk_begin(c + 1, nblk, nc);
  const uint16_t* kvb = KV + (size_t)b * N * kMlaDk;
  const size_t rows = (size_t)(gridDim.x / hg) * H;  // B * H
  const size_t row = (size_t)b * H + h0 + lq;

  if (b0 == b1) {  // an empty chunk: weight zero in the merge
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(ws_o + ((size_t)c * rows + row) * kMlaDv + 256 * half + t * 32 + g * 8 + hl * 4) = f32x4{};
    if (half == 0 && hl == 0) ws_lse[(size_t)c * rows + row] = -INFINITY;
    return;
  }
  // Q^T fragments of this wave's contraction half (B operand): lane holds
  // q[head h0 + lq][16(kh + kk) + 8hl .. +7], kh = 18 half
  const int kh = kMlaHalfK * half;
  bf16x8 qf[1][kMlaHalfK];
  {
    const uint16_t* qp = Q + row * kMlaDk + 16 * kh + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < kMlaHalfK; ++kk) {
      u32x4 raw = *(const u32x4*)(qp + kk * 16);
      if (negate_q) raw ^= 0x80008000u;
      qf[0][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  park_in_agprs<1, kMlaHalfK>(qf);
  char* xmine = smem + kMlaST * kMlaBlock + wave * 4096 + lane * 16;
  const char* xother = smem + kMlaST * kMlaBlock + (wave ^ 1) * 4096 + lane * 16;
  // row-fragment offsets: chunk 2kk + hl of row lq = 128 (kk >> 2) + 16 (2 (kk & 3) ^ e0)
  const int e0 = hl ^ (lq & 7);
  int kq[4];  // indexed by (kk - kh) & 3: step kk of this wave's half has kk & 3 = (i + (kh & 3)) & 3
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) kq[q4] = lq * kMlaRow + 16 * ((2 * ((q4 + (kh & 3)) & 3)) ^ e0);
  // transposed-read offsets (as LdsOffsets::v): row r0 + 16p + 8r, dims
  // 256 half + 32t + 16g2 + 4(ci & 3); the swizzle depends on r0 only
  const int r0 = 4 * hl + (ci >> 2), c1 = 2 * ((lane >> 4) & 1) + ((ci & 3) >> 1);
  const int tb = r0 * kMlaRow + 512 * half + 8 * (ci & 1);
  const int to0 = tb + 16 * (c1 ^ r0), to1 = tb + 16 * ((4 ^ c1) ^ r0);

  f32x16 o[1][8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[0][t] = f32x16{};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f}, alpha[1];

  // blocks j .. j+ST-2 are in flight at the top of block j; every iteration
  // issues one block's copies (past the chunk end a duplicate of its last
  // block lands in the free slot), so the count of younger copies is exact
  constexpr int PER_BLOCK = kMlaCopies / 4;
#pragma unroll
  for (int i = 0; i < kMlaST - 1; ++i)
    mla_copy_block(kvb, min(b0 + i, b1 - 1) * kMlaBN, N, smem + i * kMlaBlock, wave, lane);
  for (int j = b0; j < b1; ++j) {
    const int jr = j - b0;
    wait_vmcnt<(kMlaST - 2) * PER_BLOCK>();
    block_barrier();
    mla_copy_block(kvb, min(j + kMlaST - 1, b1 - 1) * kMlaBN, N, smem + ((jr + kMlaST - 1) % kMlaST) * kMlaBlock,
                   wave, lane);
    const char* Ks = smem + (jr % kMlaST) * kMlaBlock;
    f32x16 s[1][1];
    s[0][0] = f32x16{};
#pragma unroll
    for (int i = 0; i < kMlaHalfK; ++i) {
      const int kk = kh + i;  // runtime only through kh (0 or 18)
      s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(LDS_AS const bf16x8*)(Ks + kq[i & 3] + 128 * (kk >> 2)), qf[0][i], s[0][0], 0, 0, 0);
    }
    // swap the partial sums with the other wave of the tile
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(LDS_AS f32x4*)(xmine + g * 1024) = f32x4{s[0][0][4 * g], s[0][0][4 * g + 1], s[0][0][4 * g + 2], s[0][0][4 * g + 3]};
    block_barrier();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 o4 = *(LDS_AS const f32x4*)(xother + g * 1024);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[0][0][4 * g + e] += o4[e];
    }
    if ((j + 1) * kMlaBN > N) mask_block<kMlaBN, 1, false>(s, j * kMlaBN, 0, N, lane);
    bf16x8 pb[1][2];
    softmax_block<kMlaBN, 1>(s, pb, c_log2, m_run, l_run, alpha);
    rescale_block<256, 1>(o, alpha);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int base = ((t & 1) ? to1 : to0) + 128 * (t >> 1);
        const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Ks + base + (16 * p) * kMlaRow));
        const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Ks + base + (16 * p + 8) * kMlaRow));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][p], o[0][t], 0, 0, 0);
      }
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  const float l_tot = swap32_sum(l_run[0]);
  const float inv = 1.0f / l_tot;
  float* orow = ws_o + ((size_t)c * rows + row) * kMlaDv + 256 * half;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(orow + t * 32 + g * 8 + hl * 4) =
          f32x4{o[0][t][4 * g] * inv, o[0][t][4 * g + 1] * inv, o[0][t][4 * g + 2] * inv, o[0][t][4 * g + 3] * inv};
  if (half == 0 && hl == 0) ws_lse[(size_t)c * rows + row] = kLn2 * (m_run[0] + __builtin_amdgcn_logf(l_tot));
}

// Merge of the NC chunk partials of one (b, h) row (as attn_decode_combine,
// two output dims per thread).
__global__ __launch_bounds__(256, 1) void mla_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                                                     float* __restrict__ O, float* __restrict__ LSE, int rows, int nc) {
  __shared__ float w_sh[kDecodeMaxChunks];
  __shared__ float red[8];
  constexpr int PF = 8;  // partials per thread and dim loaded before the weights are known
  const int tid = threadIdx.x, row = blockIdx.x;
  float p0[PF], p1[PF];
#pragma unroll
  for (int c = 0; c < PF; ++c) {
    const float* src = ws_o + ((size_t)min(c, nc - 1) * rows + row) * kMlaDv;
    p0[c] = src[tid];
    p1[c] = src[tid + 256];
  }
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += 256) {
    const float l = ws_lse[(size_t)c * rows + row];
    w_sh[c] = l;
    mx = fmaxf(mx, l);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float ws = 0.f;
  for (int c = tid; c < nc; c += 256) {
    const float w = __builtin_amdgcn_exp2f((w_sh[c] - mx) * kLog2e);  // 0 for an empty chunk
    w_sh[c] = w;
    ws += w;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) ws += __shfl_xor(ws, sh);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = ws;
  __syncthreads();  // also publishes every weight in w_sh
  const float wsum = (red[4] + red[5]) + (red[6] + red[7]);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int c = 0; c < PF; ++c)
    if (c < nc) {
      a0 += w_sh[c] * p0[c];
      a1 += w_sh[c] * p1[c];
    }
  for (int c = PF; c < nc; ++c) {
    const float* src = ws_o + ((size_t)c * rows + row) * kMlaDv;
    a0 += w_sh[c] * src[tid];
    a1 += w_sh[c] * src[tid + 256];
  }
  O[(size_t)row * kMlaDv + tid] = a0 / wsum;
  O[(size_t)row * kMlaDv + tid + 256] = a1 / wsum;
  if (tid == 0) LSE[row] = mx + kLn2 * __builtin_amdgcn_logf(wsum);
}

// ---------------------------------------------------------------- host side

typedef hipError_t (*launch_fn)(const void*, const void*, const void*, float*, float*, int, int,
                                int, int, float, hipStream_t);

enum Schedule { kSimple = 0, kPipelined = 1, kPingPong = 2 };

template <int D, int NW, int BN, int QT, int SCHED, int ST, int OCC = 1>
hipError_t launch(const void* q, const void* k, const void* v, float* out, float* lse, int B,
                  int H, int N, int causal, float scale, hipStream_t stream) {
  using T = Tile<D, NW, BN, QT, ST>;
  const int n_qt = (N + T::BM - 1) / T::BM;
  const long long G = (long long)B * H * n_qt;
  const float c = fabsf(scale) * kLog2e;
  const int neg = scale < 0.f;
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  const dim3 grid((unsigned)G), block(NW * 64);
  if constexpr (SCHED == kPingPong) {
    if (causal)
      hipLaunchKernelGGL((attn_fwd_pingpong<D, NW, BN, QT, true, OCC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
    else
      hipLaunchKernelGGL((attn_fwd_pingpong<D, NW, BN, QT, false, OCC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
  } else if constexpr (SCHED == kPipelined) {
    if (causal)
      hipLaunchKernelGGL((attn_fwd_pipelined<D, NW, BN, QT, true, OCC, ST>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
    else
      hipLaunchKernelGGL((attn_fwd_pipelined<D, NW, BN, QT, false, OCC, ST>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
  } else {
    if (causal)
      hipLaunchKernelGGL((attn_fwd_simple<D, NW, BN, QT, true, ST, OCC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
    else
      hipLaunchKernelGGL((attn_fwd_simple<D, NW, BN, QT, false, ST, OCC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
  }
  return hipGetLastError();
}

struct Variant {
  const char* name;
  int d, bm, bn, waves, lds;
  launch_fn fn;
};

#define VARIANT(NAME, D, NW, BN, QT, SCHED, ST, OCC)                                   \
  Variant {                                                                            \
    NAME, D, 32 * QT * NW, BN, NW, Tile<D, NW, BN, QT, ST>::LDS_BYTES,                 \
        &launch<D, NW, BN, QT, SCHED, ST, OCC>                                         \
  }

// Name fields: head dim, query rows per workgroup, keys per block, waves,
// query tiles per wave, LDS ring slots, workgroups per CU (occ), schedule.
const Variant kVariants[] = {
    VARIANT("d64_bm256_bn64_w8_q1_st2_occ1_simple", 64, 8, 64, 1, kSimple, 2, 1),         // 0
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_simple", 128, 8, 64, 1, kSimple, 2, 1),       // 1
    VARIANT("d256_bm128_bn64_w4_q1_st2_occ1_simple", 256, 4, 64, 1, kSimple, 2, 1),       // 2
    VARIANT("d128_bm128_bn64_w4_q1_st2_occ2_simple", 128, 4, 64, 1, kSimple, 2, 2),       // 3
    VARIANT("d64_bm128_bn64_w4_q1_st2_occ2_simple", 64, 4, 64, 1, kSimple, 2, 2),         // 4
    VARIANT("d64_bm128_bn64_w4_q1_st2_occ3_simple", 64, 4, 64, 1, kSimple, 2, 3),         // 5
    VARIANT("d256_bm128_bn32_w4_q1_st2_occ2_simple", 256, 4, 32, 1, kSimple, 2, 2),       // 6
    VARIANT("d256_bm128_bn32_w4_q1_st2_occ1_simple", 256, 4, 32, 1, kSimple, 2, 1),       // 7
    VARIANT("d128_bm128_bn64_w4_q1_st3_occ1_simple", 128, 4, 64, 1, kSimple, 3, 1),       // 8
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_pingpong", 128, 8, 64, 1, kPingPong, 2, 1),   // 9
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_pipe", 128, 8, 64, 1, kPipelined, 2, 1),      // 10
    VARIANT("d64_bm256_bn64_w8_q1_st2_occ1_pipe", 64, 8, 64, 1, kPipelined, 2, 1),        // 11
    VARIANT("d128_bm256_bn64_w4_q2_st2_occ1_simple", 128, 4, 64, 2, kSimple, 2, 1),       // 12
    VARIANT("d128_bm256_bn32_w8_q1_st2_occ1_simple", 128, 8, 32, 1, kSimple, 2, 1),       // 13
    VARIANT("d128_bm256_bn32_w8_q1_st2_occ1_pipe", 128, 8, 32, 1, kPipelined, 2, 1),      // 14
    VARIANT("d64_bm128_bn32_w4_q1_st2_occ1_simple", 64, 4, 32, 1, kSimple, 2, 1),         // 15
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_pingpong", 128, 8, 128, 1, kPingPong, 2, 1), // 16
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_simple", 128, 8, 128, 1, kSimple, 2, 1),     // 17
    VARIANT("d256_bm128_bn64_w4_q1_st2_occ1_pipe", 256, 4, 64, 1, kPipelined, 2, 1),      // 18
    VARIANT("d64_bm128_bn64_w4_q1_st2_occ3_pipe", 64, 4, 64, 1, kPipelined, 2, 3),        // 19
    VARIANT("d128_bm128_bn64_w4_q1_st2_occ2_pipe", 128, 4, 64, 1, kPipelined, 2, 2),      // 20
    VARIANT("d256_bm128_bn32_w4_q1_st2_occ1_pipe", 256, 4, 32, 1, kPipelined, 2, 1),      // 21
    VARIANT("d64_bm128_bn128_w4_q1_st2_occ2_simple", 64, 4, 128, 1, kSimple, 2, 2),       // 22
    VARIANT("d128_bm256_bn32_w4_q2_st2_occ1_pipe", 128, 4, 32, 2, kPipelined, 2, 1),      // 23
    VARIANT("d128_bm256_bn32_w4_q2_st2_occ1_simple", 128, 4, 32, 2, kSimple, 2, 1),       // 24
    VARIANT("d64_bm256_bn64_w4_q2_st2_occ2_simple", 64, 4, 64, 2, kSimple, 2, 2),         // 25
    VARIANT("d64_bm256_bn128_w4_q2_st2_occ1_simple", 64, 4, 128, 2, kSimple, 2, 1),       // 26
    VARIANT("d128_bm256_bn32_w4_q2_st4_occ1_pipe", 128, 4, 32, 2, kPipelined, 4, 1),      // 27
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Measured choice per head dimension on MI355X (the same for both masks):
// the 8-wave ping-pong with 128-key blocks for d = 128; for d = 64, 4-wave
// workgroups with two query tiles per wave, two workgroups per CU; for
// d = 256, 4-wave workgroups (O alone takes 128 registers) with the in-wave
// pipelined schedule and 64-key blocks.
int default_variant(int d, int causal) {
  switch (d) {
    case 64: return 25;
    case 128: return 16;
    case 256: return 18;
    default: return -1;
  }
}

int validate(const void* q, const void* k, const void* v, const float* out, const float* lse,
             int B, int H, int N, int d, float scale, int bm) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);  // bit test: immune to fast-math folding
  if ((sbits & 0x7f800000u) == 0x7f800000u || (sbits & 0x7fffffffu) == 0) return ATTN_ERR_BAD_SCALE;
  long long bh = 0, rows = 0, elems = 0, grid = 0;
  if (__builtin_mul_overflow((long long)B, (long long)H, &bh) ||
      __builtin_mul_overflow(bh, (long long)N, &rows) ||
      __builtin_mul_overflow(rows, (long long)d, &elems) ||
      __builtin_mul_overflow(bh, (long long)((N + bm - 1) / bm), &grid))
    return ATTN_ERR_BAD_SHAPE;
  if (rows == 0) return ATTN_OK;
  // element offsets are 64-bit in the kernel; the grid is one dimension
  if (elems > (1LL << 50) || grid > INT_MAX) return ATTN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

int run_variant(int id, const void* q, const void* k, const void* v, float* out, float* lse, int B,
                int H, int N, int d, int causal, float scale, void* stream) {
  if (id < 0 || id >= kNumVariants) return ATTN_ERR_BAD_VARIANT;
  const Variant& var = kVariants[id];
  int st = validate(q, k, v, out, lse, B, H, N, d, scale, var.bm);
  if (st != ATTN_OK) return st;
  if (var.d != d) return ATTN_ERR_BAD_VARIANT;
  if (B == 0 || H == 0 || N == 0) return ATTN_OK;
  hipError_t e = var.fn(q, k, v, out, lse, B, H, N, causal, scale, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Split-KV decoding: 32-key blocks, 4 waves per workgroup (2 at d = 256,
// whose 64 KiB ring per wave fills the LDS). Each wave's K/V ring holds
// 2 slots x 2 matrices x 32 keys x d bf16, so the 160 KiB LDS of a CU keeps
// 8 waves resident at d = 64, 4 at d = 128 and 2 at d = 256; the chunks are
// sized so that one resident round of waves (256 CUs) streams the cache,
// rounded up to a multiple of the waves per workgroup.
constexpr int kDecodeBN = 32;
constexpr int kDecodeCUs = 256;
constexpr int kDecodeLdsPerCU = 160 * 1024;

constexpr int decode_waves(int d, int nw) {
  return kDecodeCUs * (kDecodeLdsPerCU / (nw * 2 * 2 * kDecodeBN * d * 2)) * nw;
}
static_assert(decode_waves(64, 4) == 2048 && decode_waves(128, 4) == 1024 && decode_waves(256, 2) == 512,
              "resident decode waves");
static_assert(decode_waves(64, 4) <= kDecodeMaxChunks, "chunk bound of the merge");

struct DecodePlan {
  int n_qt, nw, nc;
  long long rows;   // B*H*Nq
  size_t ws_bytes;  // nc * rows * (d + 1) floats
};

int decode_plan(int B, int H, int Nq, int Nkv, int d, DecodePlan* p) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  long long bh = 0, rows = 0, elems_q = 0, rows_kv = 0, elems_kv = 0;
  if (__builtin_mul_overflow((long long)B, (long long)H, &bh) ||
      __builtin_mul_overflow(bh, (long long)Nq, &rows) ||
      __builtin_mul_overflow(rows, (long long)d, &elems_q) ||
      __builtin_mul_overflow(bh, (long long)Nkv, &rows_kv) ||
      __builtin_mul_overflow(rows_kv, (long long)d, &elems_kv))
    return ATTN_ERR_BAD_SHAPE;
  p->rows = rows;
  p->nw = d == 256 ? 2 : 4;
  p->n_qt = (Nq + 31) / 32;
  p->nc = 0;
  p->ws_bytes = 0;
  if (rows == 0) return ATTN_OK;
  if (Nkv < 1) return ATTN_ERR_BAD_SHAPE;  // a query with no key has no softmax
  const long long groups = bh * p->n_qt;
  if (elems_q > (1LL << 50) || elems_kv > (1LL << 50) || groups > INT_MAX || rows > INT_MAX)
    return ATTN_ERR_BAD_SHAPE;
  const long long nblk = (Nkv + kDecodeBN - 1) / kDecodeBN;
  const long long waves = decode_waves(d, p->nw);
  long long want = (waves + groups - 1) / groups;
  if (want > nblk) want = nblk;
  const long long nc = ((want + p->nw - 1) / p->nw) * p->nw;  // <= waves <= kDecodeMaxChunks
  long long floats = 0;
  if (__builtin_mul_overflow(nc * rows, (long long)(d + 1), &floats) || floats > (1LL << 40))
    return ATTN_ERR_BAD_SHAPE;
  p->nc = (int)nc;
  p->ws_bytes = (size_t)floats * sizeof(float);
  return ATTN_OK;
}

template <int D, int NW>
hipError_t launch_decode(const DecodePlan& p, const void* q, const void* k, const void* v, float* out,
                         float* lse, int BH, int Nq, int Nkv, float scale, void* ws, hipStream_t stream) {
  const float c = fabsf(scale) * kLog2e;
  const int neg = scale < 0.f;
  float* ws_o = (float*)ws;
  float* ws_lse = ws_o + (size_t)p.nc * p.rows * D;
  const dim3 grid((unsigned)(BH * p.n_qt), (unsigned)(p.nc / NW)), block(NW * 64);
  hipLaunchKernelGGL((attn_decode_partial<D, NW, kDecodeBN>), grid, block, 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, ws_o, ws_lse, BH, Nq,
                     Nkv, p.n_qt, p.nc, c, neg);
  const int rows = (int)p.rows;
  hipLaunchKernelGGL((attn_decode_combine<D>), dim3((unsigned)rows), dim3(256), 0, stream,
                     (const float*)ws_o, (const float*)ws_lse, out, lse, rows, p.nc);
  return hipGetLastError();
}

// Backward: two waves per SIMD in both main kernels; 64-key blocks in the dQ
// kernel, 32-row query blocks in the dK/dV kernel; 32 keys or queries per
// wave. The dQ kernel runs 4 waves per workgroup. The dK/dV kernel runs 8 at
// d = 128 when that still leaves at least four workgroups per CU (each
// workgroup streams all of Q and dO once, so wider workgroups halve that
// traffic: -10% time at N = 16384), else 4 (more, smaller workgroups balance
// short causal grids better); at d = 64 a 32-row block is too small to split
// over 8 waves.
constexpr int kBwdQWaves = 4;
constexpr int kBwdCUs = 256;
constexpr int kBwdBN = 64;

struct BwdPlan {
  long long bh;
  int nqb, kw, n_ktiles, n_qtiles;
  size_t ws_bytes;  // statistics: bh * nqb * 256 bytes
};

int bwd_plan(int B, int H, int N, int d, BwdPlan* p) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  long long bh = 0, rows = 0, elems = 0;
  if (__builtin_mul_overflow((long long)B, (long long)H, &bh) || __builtin_mul_overflow(bh, (long long)N, &rows) ||
      __builtin_mul_overflow(rows, (long long)d, &elems) || elems > (1LL << 50))
    return ATTN_ERR_BAD_SHAPE;
  p->bh = bh;
  p->nqb = (N + kBwdRows - 1) / kBwdRows;
  p->kw = d == 128 && bh * ((N + 255) / 256) >= 4LL * kBwdCUs ? 8 : 4;
  p->n_ktiles = (N + 32 * p->kw - 1) / (32 * p->kw);
  p->n_qtiles = (N + 32 * kBwdQWaves - 1) / (32 * kBwdQWaves);
  if (bh * p->nqb > INT_MAX) return ATTN_ERR_BAD_SHAPE;
  p->ws_bytes = (size_t)bh * p->nqb * kBwdStatBytes;
  return ATTN_OK;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const float* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv, int N, float scale,
                      void* ws, hipStream_t stream) {
  float* stats = (float*)ws;
  // as in the forward, a negative scale negates one operand of S exactly, so
  // that c = |scale| log2e keeps -inf masks at -inf
  const float c = fabsf(scale) * kLog2e;
  const int neg = scale < 0.f;
  const unsigned gp = (unsigned)(p.bh * p.nqb);
  const unsigned gk = (unsigned)(p.bh * p.n_ktiles), gq = (unsigned)(p.bh * p.n_qtiles);
  hipLaunchKernelGGL((attn_bwd_prep<D>), dim3(gp), dim3(256), 0, stream, o, (const uint16_t*)dout, lse, stats, N,
                     p.nqb);
  if (D == 128 && p.kw == 8)
    hipLaunchKernelGGL((attn_bwd_dkdv<D, D == 128 ? 8 : 4, CAUSAL>), dim3(gk), dim3(512), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       (const float*)stats, dk, dv, N, p.n_ktiles, c, neg, scale);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv<D, 4, CAUSAL>), dim3(gk), dim3(256), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       (const float*)stats, dk, dv, N, p.n_ktiles, c, neg, scale);
  hipLaunchKernelGGL((attn_bwd_dq<D, kBwdQWaves, kBwdBN, CAUSAL>), dim3(gq), dim3(kBwdQWaves * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                     (const float*)stats, dq, N, p.n_qtiles, c, neg, scale);
  return hipGetLastError();
}

// ChunkScan: P = 64 channels per head; chunk length a multiple of 32, at most
// 256; a workgroup of four waves covers kCsRows rows of a chunk.
constexpr int kCsRows = 128;
int chunk_scan_check(int B, int S, int H, int P, int L, long long* groups) {
  if (B < 0 || S < 0 || H < 1) return ATTN_ERR_BAD_SHAPE;
  if (P != kCsP) return ATTN_ERR_HEAD_DIM;
  if (L < kCsBK || L > 256 || L % kCsBK != 0) return ATTN_ERR_BAD_SHAPE;
  long long rows = 0, elems = 0, g = 0;
  const long long nc = ((long long)S + L - 1) / L;
  if (__builtin_mul_overflow((long long)B * S, (long long)H, &rows) || __builtin_mul_overflow(rows, (long long)P, &elems) ||
      elems > (1LL << 50) || __builtin_mul_overflow((long long)B * nc, (long long)H, &g) || g > INT_MAX ||
      (long long)H * P * 2 * kCsBK > INT_MAX)
    return ATTN_ERR_BAD_SHAPE;
  *groups = g;
  return ATTN_OK;
}

// MLA decoding: H a multiple of 64 (64 heads per workgroup); chunks sized so
// that one resident round of workgroups (one per CU) covers the cache, at
// least two 32-row blocks per chunk.
struct MlaPlan {
  int nc;
  long long groups, rows;
  size_t ws_bytes;  // nc * rows * (Dv + 1) floats
};

int mla_plan(int B, int H, int N, MlaPlan* p) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (H % 64 != 0) return ATTN_ERR_BAD_SHAPE;
  p->rows = (long long)B * H;
  p->groups = (long long)B * (H / 64);
  p->nc = 0;
  p->ws_bytes = 0;
  if (p->rows == 0) return ATTN_OK;
  if (N < 1) return ATTN_ERR_BAD_SHAPE;
  long long elems = 0;
  if (__builtin_mul_overflow((long long)B * N, (long long)kMlaDk, &elems) || elems > (1LL << 50) ||
      p->rows > INT_MAX)
    return ATTN_ERR_BAD_SHAPE;
  const long long nblk = (N + kMlaBN - 1) / kMlaBN;
  long long nc = (256 + p->groups - 1) / p->groups;  // one resident round (one workgroup per CU)
  nc = std::min(nc, std::max(1LL, nblk / 2));  // at least two blocks per chunk
  nc = std::min(nc, (long long)kDecodeMaxChunks);
  long long floats = 0;
  if (__builtin_mul_overflow(nc * p->rows, (long long)(kMlaDv + 1), &floats) || floats > (1LL << 40) ||
      p->groups > INT_MAX)
    return ATTN_ERR_BAD_SHAPE;
  p->nc = (int)nc;
  p->ws_bytes = (size_t)floats * sizeof(float);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
             int N, int d, int causal, float scale, void* stream) {
  const int id = default_variant(d, causal);
  if (id < 0) {
    // still report shape errors first, as documented
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
    return ATTN_ERR_HEAD_DIM;
  }
  return run_variant(id, q, k, v, out, lse, B, H, N, d, causal, scale, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "null pointer argument";
    case ATTN_ERR_BAD_SHAPE: return "bad shape (negative size or size overflow)";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (need 64, 128 or 256)";
    case ATTN_ERR_BAD_SCALE: return "scale must be finite and nonzero";
    case ATTN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_BAD_VARIANT: return "bad kernel variant id for this head dimension";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_decode_workspace_size reports";
    default: return "unknown status";
  }
}

int attn_num_variants(void) { return kNumVariants; }

const char* attn_variant_name(int id) {
  return (id >= 0 && id < kNumVariants) ? kVariants[id].name : nullptr;
}

int attn_variant_info(int id, int* head_dim, int* block_m, int* block_n, int* waves,
                      int* lds_bytes) {
  if (id < 0 || id >= kNumVariants) return ATTN_ERR_BAD_VARIANT;
  const Variant& v = kVariants[id];
  if (head_dim) *head_dim = v.d;
  if (block_m) *block_m = v.bm;
  if (block_n) *block_n = v.bn;
  if (waves) *waves = v.waves;
  if (lds_bytes) *lds_bytes = v.lds;
  return ATTN_OK;
}

int attn_default_variant(int d, int causal) { return default_variant(d, causal); }

int attn_fwd_variant(int id, const void* q, const void* k, const void* v, float* out, float* lse,
                     int B, int H, int N, int d, int causal, float scale, void* stream) {
  return run_variant(id, q, k, v, out, lse, B, H, N, d, causal, scale, stream);
}

int attn_decode_workspace_size(int B, int H, int Nq, int Nkv, int d, size_t* bytes) {
  DecodePlan p;
  const int st = decode_plan(B, H, Nq, Nkv, d, &p);
  if (st == ATTN_OK && bytes) *bytes = p.ws_bytes;
  return st;
}

int attn_fwd_decode(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
                    int Nq, int Nkv, int d, float scale, void* workspace, size_t workspace_bytes,
                    void* stream) {
  DecodePlan p;
  int st = decode_plan(B, H, Nq, Nkv, d, &p);
  if (st != ATTN_OK) return st;
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);
  if ((sbits & 0x7f800000u) == 0x7f800000u || (sbits & 0x7fffffffu) == 0) return ATTN_ERR_BAD_SCALE;
  if (p.rows == 0) return ATTN_OK;
  if (!q || !k || !v || !out || !lse || !workspace) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)workspace;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  const int BH = B * H;
  hipError_t e;
  switch (d) {
    case 64: e = launch_decode<64, 4>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, workspace, (hipStream_t)stream); break;
    case 128: e = launch_decode<128, 4>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, workspace, (hipStream_t)stream); break;
    default: e = launch_decode<256, 2>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, workspace, (hipStream_t)stream); break;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  BwdPlan p;
  const int st = bwd_plan(B, H, N, d, &p);
  if (st == ATTN_OK && bytes) *bytes = p.ws_bytes;
  return st;
}

int attn_bwd(const void* q, const void* k, const void* v, const float* out, const float* lse, const void* dout,
             float* dq, float* dk, float* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
             size_t workspace_bytes, void* stream) {
  BwdPlan p;
  const int st = bwd_plan(B, H, N, d, &p);
  if (st != ATTN_OK) return st;
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);
  if ((sbits & 0x7f800000u) == 0x7f800000u || (sbits & 0x7fffffffu) == 0) return ATTN_ERR_BAD_SCALE;
  if (p.bh == 0 || N == 0) return ATTN_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout |
                      (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  hipError_t e;
  const hipStream_t sm = (hipStream_t)stream;
  if (d == 64)
    e = causal ? launch_bwd<64, true>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm)
               : launch_bwd<64, false>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm);
  else
    e = causal ? launch_bwd<128, true>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm)
               : launch_bwd<128, false>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int chunk_scan(const void* x, const void* cb, const float* dt, const float* dA_cumsum, float* out, int B, int S,
               int H, int P, int L, void* stream) {
  long long groups = 0;
  const int st = chunk_scan_check(B, S, H, P, L, &groups);
  if (st != ATTN_OK) return st;
  if (groups == 0) return ATTN_OK;
  if (!x || !cb || !dt || !dA_cumsum || !out) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)x | (uintptr_t)cb | (uintptr_t)dt | (uintptr_t)dA_cumsum | (uintptr_t)out;
  if ((m & 15) != 0) return ATTN_ERR_MISALIGNED;
  const int nc = (S + L - 1) / L;
  const long long parts = (L + kCsRows - 1) / kCsRows;
  if (groups * parts > INT_MAX) return ATTN_ERR_BAD_SHAPE;
  hipLaunchKernelGGL((chunk_scan_fwd<4, kCsRows / 128>), dim3((unsigned)(groups * parts)), dim3(256), 0,
                     (hipStream_t)stream,
                     (const uint16_t*)x, (const uint16_t*)cb, dt, dA_cumsum, out, S, H, L, nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int mla_decode_workspace_size(int B, int H, int N, size_t* bytes) {
  MlaPlan p;
  const int st = mla_plan(B, H, N, &p);
  if (st == ATTN_OK && bytes) *bytes = p.ws_bytes;
  return st;
}

int mla_decode(const void* q, const void* kv, float* out, float* lse, int B, int H, int N, float scale,
               void* workspace, size_t workspace_bytes, void* stream) {
  MlaPlan p;
  const int st = mla_plan(B, H, N, &p);
  if (st != ATTN_OK) return st;
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);
  if ((sbits & 0x7f800000u) == 0x7f800000u || (sbits & 0x7fffffffu) == 0) return ATTN_ERR_BAD_SCALE;
  if (p.rows == 0) return ATTN_OK;
  if (!q || !kv || !out || !lse || !workspace) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)kv | (uintptr_t)out | (uintptr_t)workspace;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)p.nc * p.rows * kMlaDv;
  hipLaunchKernelGGL(mla_decode_partial, dim3((unsigned)p.groups, (unsigned)p.nc), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)kv, ws_o, ws_lse, N, H, p.nc, fabsf(scale) * kLog2e,
                     (int)(scale < 0.f));
  hipLaunchKernelGGL(mla_combine, dim3((unsigned)p.rows), dim3(256), 0, (hipStream_t)stream, (const float*)ws_o,
                     (const float*)ws_lse, out, lse, (int)p.rows, p.nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
