// mla_decode.hip -- MLA decoding (mla_decode) on MI355X (gfx950).
//
// Part of libattn.so; the C ABI is declared in include/attn.h.

#include "attn_common.h"

namespace {

// ---------------------------------------------------------------- MLA decoding
// Multi-head latent attention decoding in the absorbed form (the decoding
// operator the PipeThreader summary page's "Discussion" paragraph cites,
// written there in about 80 lines against 500-plus by hand): all H query
// heads of a sequence attend to one shared cache of latent rows of Dk = 576
// values (512 latent + 64 rotary); a row's first Dv = 512 values are its
// value. Split over key chunks like attn_fwd_decode (normalised partials
// merged by LSE weights). A workgroup serves 64 heads, so each cache block is
// read from HBM once per 64 heads (and the H/64 workgroups of one chunk run
// on one XCD, so the second finds the block in L2). One LDS image of a
// 64-row block serves both S^T = K Q^T (row fragments) and O^T += V^T P^T
// (transposed reads of its first 512 columns). Four waves: wave = 2*tile +
// half takes the 32 heads of its tile; for S it takes rows [32 half, 32 half
// + 32) of the block with the whole 576-wide contraction (its heads' Q^T
// parked in AGPRs), for O^T the output dims [256 half, 256 half + 256) over
// all 64 rows. The two waves of a tile agree on each block's max through LDS,
// then swap their bf16 P^T halves: both hold the same softmax state.
constexpr int kMlaDk = 576, kMlaDv = 512, kMlaBN = 64;
constexpr int kMlaRow = kMlaDk * 2;             // bytes per cache row
constexpr int kMlaBlock = kMlaBN * kMlaRow;     // 72 KiB per 64-row block
constexpr int kMlaCopies = kMlaBlock / 1024;    // 1 KiB copies per block (18 per wave)
constexpr int kMlaK = kMlaDk / 16;              // 16-wide contraction steps (36)
constexpr int kMlaST = 2;                       // ring slots: one block in flight behind the one in use
constexpr int kMlaXP = 2 * 64 * 16;             // P^T exchange: two bf16x8 per lane
constexpr int kMlaXchg = 4 * (kMlaXP + 64 * 4);  // per wave: P^T, and one float per lane (max, then l)
constexpr int kMlaDummy = 4 * 256;                // L2-prefetch landing words, one per lane
// fragment reads in flight ahead of the MFMAs (one wave per SIMD: nothing
// else hides the LDS latency)
constexpr int kMlaPfQK = 8, kMlaPfPV = 4;

// 16-byte chunk c of row `row` sits at chunk (c & ~7) | ((c ^ f(row)) & 7),
// f(row) = 4 ((row >> 1) & 1) + ((row >> 2) & 3): an XOR inside each group of
// eight chunks (a row has 72), an involution. A row is 4.5 bank lines long,
// so rows of one parity share bank halves; f takes all 8 values over the
// even (and the odd) rows of any 16 consecutive rows (row-fragment reads
// conflict-free), and rows b and b + 2 (b a multiple of 4) differ in bit 2
// (the 4-row x 4-chunk transposed reads conflict-free).
__device__ __forceinline__ int mla_swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int mla_phys(int c, int row) { return (c & ~7) | ((c ^ mla_swz(row)) & 7); }

// A block's rows [row0, min(row0 + 64, N)) as a buffer resource (reads past
// them return zeros), and copy t (of 18 per wave) of the block into an LDS
// image: 1 KiB per copy, lane l's 16 bytes at dst + 1024 (4t + wave) + 16 l.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mla_rsrc(const uint16_t* kvb, int row0, int N) {
  const int rows = __builtin_amdgcn_readfirstlane(min(N - row0, kMlaBN));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(kvb + (size_t)row0 * kMlaDk), (short)0, rows * kMlaRow,
                                           kRsrcWord3);
}
__device__ __forceinline__ void mla_copy_one(__amdgpu_buffer_rsrc_t r, int t, char* dst, int wave, int lane) {
  const int pidx = (t * 4 + wave) * 64 + lane;
  const int row = pidx / 72, pc = pidx % 72;
  cs_dma(r, row * kMlaRow + (mla_phys(pc, row) << 4), dst + (t * 4 + wave) * 1024);
}
__device__ __forceinline__ void mla_copy_block(const uint16_t* kvb, int row0, int N, char* dst, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = mla_rsrc(kvb, row0, N);
#pragma unroll
  for (int t = 0; t < kMlaCopies / 4; ++t) mla_copy_one(r, t, dst, wave, lane);
}

// L2 prefetch of a block: one 4-byte read per 64-byte line of its rows, each
// landing in a throwaway LDS word of the wave (an LDS-bound load, so it ties
// up no register). With one block in flight in the LDS ring, the copy of the
// next block then finds its lines in L2 instead of waiting on HBM.
constexpr int kMlaTouch = (kMlaBlock / 64 + 255) / 256;  // reads per wave per block (5)
__device__ __forceinline__ void mla_touch_block(const uint16_t* kvb, int row0, int N, char* dummy, int wave,
                                                int lane) {
  const int rows = __builtin_amdgcn_readfirstlane(min(N - row0, kMlaBN));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(kvb + (size_t)row0 * kMlaDk), (short)0,
                                                                     rows * kMlaRow, kRsrcWord3);
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)dummy;
#pragma unroll
  for (int t = 0; t < kMlaTouch; ++t) {
    const int voff = ((t * 4 + wave) * 64 + lane) * 64;  // past the block: the range check reads nothing
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
                 "s"(m0)
                 : "m0", "memory");
  }
}

// Grid: B * (H/64) * NC workgroups. Chunk c of the key blocks as chunk_begin.
__global__ __launch_bounds__(256, 1) void mla_decode_partial(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ KV,
                                                            float* __restrict__ ws_o, float* __restrict__ ws_lse,
                                                            int N, int H, int nc, float c_log2, int q_mode) {
  static_assert(kMlaCopies % 4 == 0, "copies split evenly over four waves");
  __shared__ __attribute__((aligned(1024))) char smem[kMlaST * kMlaBlock + kMlaXchg + kMlaDummy];
  const int lane = threadIdx.x & 63, hl = lane >> 5, lq = lane & 31, ci = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = wave >> 1, half = wave & 1;
  // The H/64 head groups of one (sequence, chunk) take consecutive logical
  // ids, which xcd_remap places on one XCD at once: the group that fetches a
  // cache block second finds it in that XCD's L2.
  const int hg = H / 64;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hgi = L % hg, bc = L / hg;
  const int b = bc / nc, c = bc % nc, h0 = hgi * 64 + 32 * tile;
  const int nblk = (N + kMlaBN - 1) / kMlaBN;
  const int b0 = chunk_begin(c, nblk, nc), b1 = chunk_begin(c + 1, nblk, nc);
  const uint16_t* kvb = KV + (size_t)b * N * kMlaDk;
  const size_t rows = (size_t)(gridDim.x / (hg * nc)) * H;  // B * H
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
  char* xbase = smem + kMlaST * kMlaBlock;
  char* xp_mine = xbase + wave * kMlaXP + lane * 16;
  const char* xp_other = xbase + (wave ^ 1) * kMlaXP + lane * 16;
  float* xf_mine = (float*)(xbase + 4 * kMlaXP) + wave * 64 + lane;
  const float* xf_other = (const float*)(xbase + 4 * kMlaXP) + (wave ^ 1) * 64 + lane;
  // row-fragment offsets: row 32 half + lq, chunk 2kk + hl at
  // 128 (kk >> 2) + 16 ((2 (kk & 3)) ^ hl ^ mla_swz(lq))  (mla_swz(32 m + lq) = mla_swz(lq))
  const int e0 = hl ^ mla_swz(lq);
  int kq[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) kq[q4] = (32 * half + lq) * kMlaRow + 16 * ((2 * q4) ^ e0);
  // transposed-read offsets (as LdsOffsets::v): rows r0 + 16p + 8r of a 32-row
  // key tile, dims 256 half + 32t + 16g2 + 4(ci & 3); the swizzle of row
  // r0 + 8r + 16p + 32kt is mla_swz(r0) ^ 2r (r0 < 8)
  const int r0 = 4 * hl + (ci >> 2), c1 = 2 * ((lane >> 4) & 1) + ((ci & 3) >> 1);
  const int tb = r0 * kMlaRow + 512 * half + 8 * (ci & 1), f0 = mla_swz(r0);
  int to[2][2];  // [t & 1][r]
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    to[0][r] = tb + 16 * (c1 ^ f0 ^ (2 * r)) + 8 * r * kMlaRow;
    to[1][r] = tb + 16 * ((4 ^ c1) ^ f0 ^ (2 * r)) + 8 * r * kMlaRow;
  }
  const int vrow_mine = 32 * half * kMlaRow, vrow_other = 32 * (half ^ 1) * kMlaRow;

  f32x16 o[1][8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[0][t] = f32x16{};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f}, alpha[1];

  // The 64 heads' Q rows are contiguous: they go to ring slot 1 as a 64-row
  // block (same layout) while block b0 goes to slot 0. Each iteration then
  // issues the next block's copies, and the L2 prefetch of the block after
  // (past the chunk end: duplicates of its last block, so the count of
  // younger loads at the top of a block is always kMlaTouch).
  char* dummy = smem + kMlaST * kMlaBlock + kMlaXchg + wave * 256;
  mla_copy_block(Q + ((size_t)b * H + hgi * 64) * kMlaDk, 0, kMlaBN, smem + kMlaBlock, wave, lane);
  mla_copy_block(kvb, b0 * kMlaBN, N, smem, wave, lane);
  mla_touch_block(kvb, min(b0 + 1, b1 - 1) * kMlaBN, N, dummy, wave, lane);
  wait_vmcnt<kMlaCopies / 4 + kMlaTouch>();  // the Q copies, issued first, have landed
  block_barrier();
  // Q^T fragments (B operand): lane holds q[head h0 + lq][16 kk + 8 hl .. +7],
  // row 32 tile + lq of the Q image; slot 1 is refilled only after the
  // barrier at the top of the first block
  bf16x8 qf[1][kMlaK];
  {
    const char* qimg = smem + kMlaBlock + (32 * tile - 32 * half) * kMlaRow;
#pragma unroll
    for (int kk = 0; kk < kMlaK; ++kk) {
      u32x4 raw = *(LDS_AS const u32x4*)(qimg + kq[kk & 3] + 128 * (kk >> 2));
      raw = apply_q_mode(raw, q_mode);
      qf[0][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  park_in_agprs<1, kMlaK>(qf);
  for (int j = b0; j < b1; ++j) {
    const int slot = (j - b0) & 1;
    wait_vmcnt<kMlaTouch>();
    block_barrier();
    // the next block's 18 copies are spread over this block's 68 MFMAs (9 in
    // the QK stream, 9 in the PV stream): issued together they hold the wave
    // at the texture unit for about a fifth of the block
    const __amdgpu_buffer_rsrc_t rnext = mla_rsrc(kvb, min(j + 1, b1 - 1) * kMlaBN, N);
    char* cdst = smem + (slot ^ 1) * kMlaBlock;
    const char* Ks = smem + slot * kMlaBlock;
    const int kv0 = j * kMlaBN + 32 * half;
    f32x16 s[1][1];
    if (kv0 < N) {  // wave-uniform: the second half of the last block may hold no key
      // two accumulator chains (even and odd steps); fragments read
      // kMlaPfQK steps ahead
      f32x16 s2[2] = {f32x16{}, f32x16{}};
      bf16x8 kf[kMlaPfQK];
#pragma unroll
      for (int i = 0; i < kMlaPfQK; ++i) kf[i] = *(LDS_AS const bf16x8*)(Ks + kq[i & 3] + 128 * (i >> 2));
#pragma unroll
      for (int kk = 0; kk < kMlaK; ++kk) {
        s2[kk & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % kMlaPfQK], qf[0][kk], s2[kk & 1], 0, 0, 0);
        if (kk + kMlaPfQK < kMlaK) {
          const int kn = kk + kMlaPfQK;
          kf[kk % kMlaPfQK] = *(LDS_AS const bf16x8*)(Ks + kq[kn & 3] + 128 * (kn >> 2));
        }
        if ((kk & 3) == 3) mla_copy_one(rnext, kk >> 2, cdst, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      s[0][0] = s2[0] + s2[1];
      if (kv0 + 32 > N) mask_block<32, 1, false>(s, kv0, 0, N, lane);
    } else {
#pragma unroll
      for (int t = 0; t < 9; ++t) mla_copy_one(rnext, t, cdst, wave, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[0][0][r] = -INFINITY;
    }
    // the block max of each head over both halves (exact), then the common
    // running max; c > 0, so fl(max(s) c) = max(fl(s c))
    float mx = fmaxf(fmaxf(s[0][0][0], s[0][0][1]), s[0][0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[0][0][r]), s[0][0][r + 1]);
    mx = swap32_max(fmaxf(mx, s[0][0][15]));
    *xf_mine = mx;
    block_barrier();
    const float m_new = fmaxf(m_run[0], fmaxf(mx, *xf_other) * c_log2);
    alpha[0] = __builtin_amdgcn_exp2f(m_run[0] - m_new);
    m_run[0] = m_new;
    float ps[1][4];
    softmax_exp<32, 1, 0>(s, c_log2, m_run, ps);
    bf16x8 pb[1][2];
    softmax_pack<32, 1>(s, pb);
    softmax_sum<1>(l_run, alpha, ps);
    *(LDS_AS bf16x8*)(xp_mine) = pb[0][0];
    *(LDS_AS bf16x8*)(xp_mine + 64 * 16) = pb[0][1];
    block_barrier();
    // P^T of this wave's key tile (rows 32 half ..) and of the partner's
    // (rows 32 (half ^ 1) ..): own tile first, so that every operand index is
    // a compile-time constant
    bf16x8 pt[2][2];
    pt[0][0] = pb[0][0];
    pt[0][1] = pb[0][1];
    pt[1][0] = *(LDS_AS const bf16x8*)(xp_other);
    pt[1][1] = *(LDS_AS const bf16x8*)(xp_other + 64 * 16);
    rescale_block<256, 1>(o, alpha);
    // PV step i = 16 kt + 8 p + t: O^T tile t += V^T(key tile kt, rows 16p..) P^T;
    // the transposed reads run kMlaPfPV steps ahead, and copies 9-17 of the
    // next block go out at steps 1, 5, .., 29 and 31
    auto tr_read = [&](int i, i16x4& a0, i16x4& a1) {
      const int kt = i >> 4, p = (i >> 3) & 1, t = i & 7;
      const int base = 128 * (t >> 1) + (kt ? vrow_other : vrow_mine) + (16 * p) * kMlaRow;
      a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Ks + base + to[t & 1][0]));
      a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(Ks + base + to[t & 1][1]));
    };
    i16x4 va[kMlaPfPV][2];
#pragma unroll
    for (int i = 0; i < kMlaPfPV; ++i) tr_read(i, va[i][0], va[i][1]);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int kt = i >> 4, p = (i >> 3) & 1, t = i & 7;
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[i % kMlaPfPV][0], va[i % kMlaPfPV][1], 0, 1, 2, 3, 4,
                                                             5, 6, 7));
      o[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pt[kt][p], o[0][t], 0, 0, 0);
      if (i + kMlaPfPV < 32) tr_read(i + kMlaPfPV, va[i % kMlaPfPV][0], va[i % kMlaPfPV][1]);
      if ((i & 3) == 1 || i == 31) mla_copy_one(rnext, i == 31 ? 17 : 9 + (i >> 2), cdst, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    // issued after every copy of the next block, so that at the top of the
    // next block only these kMlaTouch reads may still be in flight
    mla_touch_block(kvb, min(j + 2, b1 - 1) * kMlaBN, N, dummy, wave, lane);
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  // the row sum: this wave's keys, then the partner's (same alpha sequence)
  const float l_mine = swap32_sum(l_run[0]);
  block_barrier();  // the partner has read this wave's last max
  *xf_mine = l_mine;
  block_barrier();
  const float l_tot = l_mine + *xf_other;
  const float inv = 1.0f / l_tot;
  // O^T (lane = head, registers = dims) goes through LDS so that each store
  // writes one head's 256 dims (1 KiB) contiguously: [head][dim] per wave,
  // 16-byte chunk k of row h at k ^ (h & 15) (conflict-free both ways)
  char* st = smem + wave * (32 * 1024);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(LDS_AS f32x4*)(st + lq * 1024 + (((8 * t + 2 * g + hl) ^ (lq & 15)) << 4)) =
          f32x4{o[0][t][4 * g] * inv, o[0][t][4 * g + 1] * inv, o[0][t][4 * g + 2] * inv, o[0][t][4 * g + 3] * inv};
  // (a wave reads back only its own rows; its LDS accesses complete in order)
  float* obase = ws_o + ((size_t)c * rows + (size_t)b * H + h0) * kMlaDv + 256 * half;
#pragma unroll 4
  for (int h = 0; h < 32; ++h)
    *(f32x4*)(obase + (size_t)h * kMlaDv + 4 * lane) = *(LDS_AS const f32x4*)(st + h * 1024 + ((lane ^ (h & 15)) << 4));
  if (half == 0 && hl == 0) ws_lse[(size_t)c * rows + row] = kLn2 * (m_run[0] + __builtin_amdgcn_logf(l_tot));
}

// Merge of the NC chunk partials of one (b, h) row, for NC <= kMlaMergePF
// (many rows, few chunks): one wave per row, four rows per workgroup, lane l owning output dims 8l .. 8l + 7. Every lane reads
// all NC chunk LSEs (the same addresses in every lane: one request each) and
// its 8 dims of every partial, all issued before any weight is known, so the
// merge costs one memory round trip; no barrier. (Few rows with many chunks
// go to mla_combine_wide instead.) Weights and sums run over the
// chunks in order: w_c = exp(LSE_c - max), O = sum w_c O_c / sum w_c,
// LSE = max + ln(sum w_c) (an empty chunk has LSE -inf and weight 0).
constexpr int kMlaMergePF = 8;  // chunks whose partials are loaded up front
__global__ __launch_bounds__(256) void mla_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                                                   float* __restrict__ O, float* __restrict__ LSE, int rows, int nc) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  f32x4 p0[kMlaMergePF], p1[kMlaMergePF];
  float lse[kMlaMergePF];
#pragma unroll
  for (int c = 0; c < kMlaMergePF; ++c) {
    // past the last chunk: a duplicate of it (an L2 hit), never weighted;
    // guarding the loads instead makes the compiler keep every slot live
    const int cc = min(c, nc - 1);
    const float* src = ws_o + ((size_t)cc * rows + row) * kMlaDv + 8 * lane;
    p0[c] = *(const f32x4*)src;
    p1[c] = *(const f32x4*)(src + 4);
    lse[c] = ws_lse[(size_t)cc * rows + row];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < kMlaMergePF; ++c)
    if (c < nc) mx = fmaxf(mx, lse[c]);
  float wsum = 0.f;
  f32x4 a0 = f32x4{}, a1 = f32x4{};
#pragma unroll
  for (int c = 0; c < kMlaMergePF; ++c)
    if (c < nc) {
      const float w = __builtin_amdgcn_exp2f((lse[c] - mx) * kLog2e);  // 0 for an empty chunk
      wsum += w;
      a0 += w * p0[c];
      a1 += w * p1[c];
    }
  const float inv = 1.0f / wsum;
  float* dst = O + (size_t)row * kMlaDv + 8 * lane;
  *(f32x4*)dst = a0 * inv;
  *(f32x4*)(dst + 4) = a1 * inv;
  if (lane == 0) LSE[row] = mx + kLn2 * __builtin_amdgcn_logf(wsum);
}

// Merge for many chunks (more than kMlaMergePF): one workgroup per row (as
// attn_decode_combine), two output dims per thread, the chunk weights shared
// through LDS.
__global__ __launch_bounds__(256, 1) void mla_combine_wide(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
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


// MLA decoding: H a multiple of 64 (64 heads per workgroup); chunks sized so
// that one resident round of workgroups (one per CU) covers the cache, at
// least two 64-row blocks per chunk (one-block chunks: B = 1 took 26.7
// against 22.5 us, the per-workgroup Q load and partial stores then
// dominate).
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
      !grid_fits(p->groups * nc, 256) || !grid_fits(p->rows, 256))
    return ATTN_ERR_BAD_SHAPE;
  p->nc = (int)nc;
  p->ws_bytes = (size_t)floats * sizeof(float);
  return ATTN_OK;
}

}  // namespace

extern "C" {

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
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_BAD_SCALE;  // NaN or +-Inf
  if (p.rows == 0) return ATTN_OK;
  if (!q || !kv || !out || !lse || !workspace) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)kv | (uintptr_t)out | (uintptr_t)workspace;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  float* ws_o = (float*)workspace;
  float* ws_lse = ws_o + (size_t)p.nc * p.rows * kMlaDv;
  clear_last_hip_error();
  hipLaunchKernelGGL(mla_decode_partial, dim3((unsigned)(p.groups * p.nc)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)kv, ws_o, ws_lse, N, H, p.nc, scale_args(scale).c_log2,
                     scale_args(scale).q_mode);
  if (p.nc <= kMlaMergePF)
    hipLaunchKernelGGL(mla_combine, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       (const float*)ws_o, (const float*)ws_lse, out, lse, (int)p.rows, p.nc);
  else
    hipLaunchKernelGGL(mla_combine_wide, dim3((unsigned)p.rows), dim3(256), 0, (hipStream_t)stream,
                       (const float*)ws_o, (const float*)ws_lse, out, lse, (int)p.rows, p.nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
