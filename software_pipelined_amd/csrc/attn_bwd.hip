// attn_bwd.hip -- attention backward (attn_bwd) on MI355X (gfx950).
//
// Part of libattn.so; the C ABI is declared in include/attn.h.

#include "attn_common.h"

namespace {

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
// (swz_dual, conflict-free for both reads) serves both as row-fragment A
// operand (ds_read_b128) and, through ds_read_b64_tr_b16, as the transposed A
// operand; an MFMA accumulator tile converted to bf16 is the B operand of the
// next product without an LDS round trip.

constexpr int kBwdRows = 32;               // query rows per statistics block
constexpr int kBwdStatBytes = 2 * kBwdRows * 4;  // log2e*LSE then D, fp32

// Compact fragment offsets into a swz_dual [rows][D] image, one or two
// registers per lane instead of one per fragment: the swizzle only permutes
// 16-byte chunks within a row, so every fragment's offset is one lane base
// XOR a compile-time constant (the row part and the chunk part occupy
// disjoint bits).
//   row fragment kk (A operand, ds_read_b128): row lq, chunk 2kk + h
//       = kbase ^ (32 kk);
//   transposed read (t, r) (ds_read_b64_tr_b16, as LdsOffsets::v): rows
//       r0 + 8r, r0 < 8; swz_dual(r0 + 8) = swz_dual(r0) ^ 2, so the second
//       base is tbase ^ 32; dims tile t = base ^ (64 t); adding 16p rows
//       leaves the swizzle unchanged.
template <int D>
struct BwdOffsets {
  int kbase, tbase;
  __device__ __forceinline__ explicit BwdOffsets(int lane) {
    const int h = lane >> 5, lq = lane & 31, ci = lane & 15, g2 = (lane >> 4) & 1;
    kbase = lq * (D * 2) + ((h ^ swz_dual<D>(lq)) << 4);
    const int r0 = 4 * h + (ci >> 2), c1 = 2 * g2 + ((ci & 3) >> 1);
    tbase = r0 * (D * 2) + ((c1 ^ swz_dual<D>(r0)) << 4) + 8 * (ci & 1);
  }
  __device__ __forceinline__ int k(int kk) const { return kbase ^ (32 * kk); }
  __device__ __forceinline__ int t(int r, int tt) const { return tbase ^ (32 * r) ^ (64 * tt); }
};

// mma_qk from a swz_dual image (as qk_block): S^T[key][query] for BN rows of
// the image against Q^T fragments held in registers.
template <int D, int BN>
__device__ __forceinline__ void qk_block_dual(const char* img, const BwdOffsets<D>& bo, const bf16x8 (&qf)[1][D / 16],
                                              f32x16 (&s)[1][BN / 32]) {
  constexpr int NKB = BN / 32;
  bf16x8 kf[D / 16][NKB];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kf[kk][kb] = *(LDS_AS const bf16x8*)(img + bo.k(kk) + kb * 32 * (D * 2));
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[0][kb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      s[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][kb], qf[0][kk], s[0][kb], 0, 0, 0);
}

// A operand of X^T[dim tile t][rows 16p .. 16p+15] from a swz_dual image.
template <int D>
__device__ __forceinline__ bf16x8 read_tr_k(const char* img, const BwdOffsets<D>& bo, int t, int p) {
  const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(img + bo.t(0, t) + (p * 16) * (D * 2)));
  const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(img + bo.t(1, t) + (p * 16 + 8) * (D * 2)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup-shared HBM -> LDS copy t of a BN-row block (placement as
// issue_copy, swz_dual), in inline assembly so that the compiler's
// conservative wait before transposed LDS reads does not drain the copies of
// the next block; callers wait with wait_vmcnt.
template <int D, int NW, int BN>
__device__ __forceinline__ void issue_copy_asm(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                               int wave, int lane, int t) {
  cs_dma(block_rsrc<D, BN>(src, row0, N), (int)block_lane_offset_sw<D, NW, BN, 2>(t, wave, lane),
         dst + (t * NW + wave) * 64 * 16);
}

// The lane index from mbcnt, in a volatile asm block the compiler can neither
// hoist nor merge: values derived from it inside the block loop are
// recomputed there each block rather than kept live across the loop. When
// such a value is spilled instead, its scratch reload at the top of a block
// comes with a vmcnt wait that also drains the next block's copies.
__device__ __forceinline__ int opaque_lane() {
  int v;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0"
      : "=v"(v));
  return v;
}

// Workgroups per CU the main kernels are compiled for: two waves per SIMD
// (256 registers each) at d = 64 and 128; one at d = 256, where a wave's
// K/V (or Q/dO) operands and its two d-wide accumulators need about 450.
constexpr int bwd_blocks_per_cu(int D, int NW) { return D == 256 ? 4 / NW : 8 / NW; }

// One 256-byte statistics block into a wave's own 1 KiB LDS slot (lanes past
// the block read zeros).
__device__ __forceinline__ void issue_stat_copy(const float* src, char* dst) {
  cs_dma(__builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, kBwdStatBytes, kRsrcWord3), opaque_lane() * 16,
         dst);
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

// Issue priority of the MFMA phases (s_setprio) at d = 64, where the per-score
// VALU work (exp2, the dS product, bf16 packing) is largest next to the MFMA
// work: with two waves per SIMD the wave in its MFMA phase then issues ahead
// of the other's VALU phase (same-host A/B: 3 % faster at d = 64; 1-3 %
// slower at d = 128 and 256, which keep equal priority).
template <int D, int P>
__device__ __forceinline__ void bwd_prio() {
  if constexpr (D == 64) __builtin_amdgcn_s_setprio(P);
}

// dK, dV. Workgroup = NW waves, wave w owns keys k0 + 32w .. +31 (K and V
// rows as B-operand registers). Query blocks of 32 rows (Q, dO, statistics)
// stream through a two-stage LDS ring. Per block and wave:
//   S = Q K^T, dP = dO V^T          (A = Q / dO row fragments, B = K / V)
//   P = exp2(c*S - log2e*LSE), dS = P (dP - D)   (accumulator layout: query rows)
//   dV^T += dO^T P, dK^T += Q^T dS  (A = transposed reads, B = P / dS in bf16)
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, bwd_blocks_per_cu(D, NW)) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ stats, float* __restrict__ dK,
    float* __restrict__ dV, int N, int n_ktiles, float c_log2, int q_mode, float scale) {
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
  load_q<D, 1>(K + head, k0w, N, q_mode, kf, lane);  // K as scale_args takes it
  load_q<D, 1>(V + head, k0w, N, 0, vf, lane);
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
    issue_stat_copy(st_head + (size_t)jb * (2 * BQ), base + 2 * MAT + wave * STAT);
  };

  const int jb0 = CAUSAL ? min(k0 / BQ, nqb) : 0;  // earlier query blocks see none of these keys
  if (jb0 < nqb) copy_stage(jb0, 0);
  for (int jb = jb0; jb < nqb; ++jb) {
    const int slot = (jb - jb0) & 1;
    wait_vmcnt<0>();
    block_barrier();
    if (jb + 1 < nqb) copy_stage(jb + 1, slot ^ 1);
    const char* Qs = smem + slot * STAGE;
    const char* dOs = Qs + MAT;
    const int q0 = jb * BQ;
    if (CAUSAL && q0 + BQ - 1 < k0w) continue;  // wave-uniform: every query precedes every key of this wave
    // d = 128: per-lane offsets rebuilt each block (opaque_lane), so nothing
    // lane-derived stays live across the loop next to the K/V operands and
    // the accumulators (256 registers with two waves per SIMD). d = 64 has
    // room and keeps them loop-invariant.
    const int ln = D >= 128 ? opaque_lane() : lane, hl = ln >> 5, key = k0w + (ln & 31);
    const BwdOffsets<D> bo(ln);
    const char* Ss = Qs + 2 * MAT + wave * STAT;
    // fragments are read right before the MFMA that consumes them: with two
    // waves per SIMD the K/V operands and dK/dV accumulators leave little room
    f32x16 s = f32x16{}, dp = f32x16{};
    bwd_prio<D, 1>();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(LDS_AS const bf16x8*)(Qs + bo.k(kk)), kf[0][kk], s, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(LDS_AS const bf16x8*)(dOs + bo.k(kk)), vf[0][kk], dp, 0, 0, 0);
    const bool diag = CAUSAL && q0 < k0w + 31;
    bwd_prio<D, 0>();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2 = *(LDS_AS const f32x4*)(Ss + (8 * g + 4 * hl) * 4);
      const f32x4 dd = *(LDS_AS const f32x4*)(Ss + BQ * 4 + (8 * g + 4 * hl) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2[i]));
        if (diag) {
          const int qi = q0 + 8 * g + 4 * hl + i;
          p = key > qi ? 0.f : p;
        }
        s[r] = p;
        dp[r] = p * (dp[r] - dd[i]);
      }
    }
    bf16x8 pb[1][2], dsb[1][2];
    softmax_pack<32, 1>(*(const f32x16(*)[1][1])&s, pb);
    softmax_pack<32, 1>(*(const f32x16(*)[1][1])&dp, dsb);
    bwd_prio<D, 1>();
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
  const int key = k0w + (lane & 31);
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
__global__ __launch_bounds__(NW * 64, bwd_blocks_per_cu(D, NW)) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ stats, float* __restrict__ dQ, int N,
    int n_qtiles, float c_log2, int q_mode, float scale) {
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
  load_q<D, 1>(Q + head, q0w, N, q_mode, qf, lane);  // Q as scale_args takes it
  load_q<D, 1>(dO + head, q0w, N, 0, gf, lane);
  const int qs = min(qi, nqb * kBwdRows - 1);  // rows past N: padded statistics (+inf, 0)
  const float* st = stats + ((size_t)bh * nqb + qs / kBwdRows) * (2 * kBwdRows);
  const float l2 = st[qs % kBwdRows], dd = st[kBwdRows + qs % kBwdRows];
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
    bwd_prio<D, 1>();
    qk_block_dual<D, BN>(Ks, bo, qf, s);
    qk_block_dual<D, BN>(Vs, bo, gf, dp);
    bwd_prio<D, 0>();
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
    bwd_prio<D, 1>();
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

// Backward: two waves per SIMD in both main kernels (one at d = 256,
// bwd_blocks_per_cu); 64-key blocks in the dQ
// kernel, 32-row query blocks in the dK/dV kernel; 32 keys or queries per
// wave. The dQ kernel runs 4 waves per workgroup. The dK/dV kernel runs 8 at
// d = 128 when that still leaves at least four workgroups per CU (each
// workgroup streams all of Q and dO once, so wider workgroups halve that
// traffic: -10% time at N = 16384), else 4 (more, smaller workgroups balance
// short causal grids better); at d = 64 a 32-row block is too small to split
// over 8 waves.
// dQ kernel waves: 8 at d = 128 without the mask (256 queries per
// workgroup, so every K/V block staged in LDS serves twice as many queries:
// -1.2 % time at N = 16384); else 4 (d = 64 keeps three 4-wave workgroups
// per CU, which 8-wave ones would cut to one: +7 % time; causal grids are
// neutral; d = 256 fits one wave per SIMD only).
constexpr int bwd_q_waves(int d, bool causal) { return d == 128 && !causal ? 8 : 4; }
constexpr int kBwdCUs = 256;
constexpr int kBwdBN = 64;

struct BwdPlan {
  long long bh;
  int nqb, kw, qw, n_ktiles, n_qtiles;
  size_t ws_bytes;  // statistics: bh * nqb * 256 bytes
};

int bwd_plan(int B, int H, int N, int d, BwdPlan* p) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  long long bh = 0, rows = 0, elems = 0;
  if (__builtin_mul_overflow((long long)B, (long long)H, &bh) || __builtin_mul_overflow(bh, (long long)N, &rows) ||
      __builtin_mul_overflow(rows, (long long)d, &elems) || elems > (1LL << 50))
    return ATTN_ERR_BAD_SHAPE;
  p->bh = bh;
  p->nqb = (N + kBwdRows - 1) / kBwdRows;
  p->kw = d == 128 && bh * ((N + 255) / 256) >= 4LL * kBwdCUs ? 8 : 4;
  p->n_ktiles = (N + 32 * p->kw - 1) / (32 * p->kw);
  p->qw = bwd_q_waves(d, false);  // attn_bwd sets the mask's value
  p->n_qtiles = (N + 32 * p->qw - 1) / (32 * p->qw);
  if (!grid_fits(bh * p->nqb, 512)) return ATTN_ERR_BAD_SHAPE;  // the largest of the three grids
  p->ws_bytes = (size_t)bh * p->nqb * kBwdStatBytes;
  return ATTN_OK;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const float* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv, int N, float scale,
                      void* ws, hipStream_t stream) {
  float* stats = (float*)ws;
  // as in the forward, the sign of the scale goes into one operand of S
  // (negated, or zeroed for a zero scale; scale_args), so that c > 0 keeps
  // -inf masks at -inf; dK and dQ are multiplied by the scale itself
  const ScaleArgs sa = scale_args(scale);
  const float c = sa.c_log2;
  const int neg = sa.q_mode;
  const unsigned gp = (unsigned)(p.bh * p.nqb);
  const unsigned gk = (unsigned)(p.bh * p.n_ktiles), gq = (unsigned)(p.bh * p.n_qtiles);
  clear_last_hip_error();
  hipLaunchKernelGGL((attn_bwd_prep<D>), dim3(gp), dim3(256), 0, stream, o, (const uint16_t*)dout, lse, stats, N,
                     p.nqb);
  if (D == 128 && p.kw == 8)
    hipLaunchKernelGGL((attn_bwd_dkdv<D, D == 128 ? 8 : 4, CAUSAL>), dim3(gk), dim3(512), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       (const float*)stats, dk, dv, N, p.n_ktiles, c, neg, scale);
  else  // 4 waves: d = 64, d = 256, and d = 128 on small grids
    hipLaunchKernelGGL((attn_bwd_dkdv<D, 4, CAUSAL>), dim3(gk), dim3(256), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                       (const float*)stats, dk, dv, N, p.n_ktiles, c, neg, scale);
  constexpr int QW = bwd_q_waves(D, CAUSAL);
  hipLaunchKernelGGL((attn_bwd_dq<D, QW, kBwdBN, CAUSAL>), dim3(gq), dim3(QW * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                     (const float*)stats, dq, N, p.n_qtiles, c, neg, scale);
  return hipGetLastError();
}

}  // namespace

extern "C" {

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
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_BAD_SCALE;  // NaN or +-Inf
  if (p.bh == 0 || N == 0) return ATTN_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout |
                      (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  p.qw = bwd_q_waves(d, causal != 0);
  p.n_qtiles = (N + 32 * p.qw - 1) / (32 * p.qw);
  hipError_t e;
  const hipStream_t sm = (hipStream_t)stream;
  if (d == 64)
    e = causal ? launch_bwd<64, true>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm)
               : launch_bwd<64, false>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm);
  else if (d == 128)
    e = causal ? launch_bwd<128, true>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm)
               : launch_bwd<128, false>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm);
  else
    e = causal ? launch_bwd<256, true>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm)
               : launch_bwd<256, false>(p, q, k, v, out, lse, dout, dq, dk, dv, N, scale, workspace, sm);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
