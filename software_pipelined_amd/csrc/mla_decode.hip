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
// (transposed reads of its first 512 columns). Eight waves, two per SIMD,
// on v_mfma_f32_16x16x32_bf16 tiles of 16 heads: wave = 2*tile + half takes
// the 16 heads of its tile; for S it takes rows [32 half, 32 half + 32) of
// the block (two 16-key tiles) with the whole 576-wide contraction (its
// heads' Q^T, 18 fragments, in registers), for O^T the output dims
// [256 half, 256 half + 256) (16 tiles of 16) over all 64 rows. The two
// waves of a tile agree on each block's max through LDS, then swap their
// bf16 P^T halves: both hold the same softmax state.
//
// The P^T operand of the PV step is the S accumulator as it stands: lane l
// holds keys 4g + i and 16 + 4g + i (g = l >> 4, i < 4) of its head l & 15,
// which become contraction indices 8g + i and 8g + 4 + i of the 32-key step;
// the V^T operand reads its rows in that same order (two transposed reads,
// rows 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3).
//
// With few sequences the same kernel runs on workgroups of one head tile
// (16 heads, two waves; MlaShape<1>), so that the grid still covers the CUs.
typedef float f32x8 __attribute__((ext_vector_type(8)));
constexpr int kMlaDk = 576, kMlaDv = 512, kMlaBN = 64;
constexpr int kMlaRow = kMlaDk * 2;                // bytes per cache row
constexpr int kMlaBlock = kMlaBN * kMlaRow;        // 72 KiB per 64-row block
constexpr int kMlaCopies = kMlaBlock / 1024;       // 1 KiB copies per block
constexpr int kMlaK = kMlaDk / 32;                 // 32-wide contraction steps (18)
constexpr int kMlaST = 2;                          // ring slots: one block in flight behind the one in use
constexpr int kMlaXP = 64 * 16;                    // P^T exchange: one bf16x8 per lane

// A workgroup of T head tiles (16 heads each) and 2T waves: T = 4 (64 heads,
// eight waves, two per SIMD) by default; T = 1 (16 heads, two waves) when
// 64-head workgroups would leave CUs idle (few sequences: B = 1 fills 64 of
// 256 CUs with them, all 256 with 16-head ones).
template <int T>
struct MlaShape {
  static constexpr int W = 2 * T;                        // waves
  static constexpr int HEADS = 16 * T;
  static constexpr int CPW = kMlaCopies / W;             // 1 KiB copies per wave and block (9 or 36)
  static constexpr int SC = T == 4 ? 7 : CPW;            // of them, issued in the S stream
  static constexpr int XCHG = W * (kMlaXP + 64 * 4);     // per wave: P^T, and one float per lane (max, then l)
  // the copy issued at S-stream step i (of 36) and at PV-stream step i (of
  // 32), or -1: with T = 4 one per five S steps and the last two early in
  // the PV stream; with T = 1 one per S step
  static constexpr int s_copy(int i) { return T == 4 ? (i % 5 == 1 ? i / 5 : -1) : (i < CPW ? i : -1); }
  static constexpr int pv_copy(int i) { return T == 4 && (i & 7) == 1 && i < 16 ? SC + (i >> 3) : -1; }
  static_assert(kMlaCopies % W == 0, "copies split evenly over the waves");
};
// fragment reads in flight ahead of the MFMAs (a PV step takes two
// transposed reads)
constexpr int kMlaPfQK = 6, kMlaPfPV = 8;

// 16-byte chunk c of row `row` sits at chunk c ^ f(row) (f < 8: an XOR
// inside each group of eight chunks; a row has 72), with x = (row >> 1) & 7,
// h = (x & 1) + 2 (((x >> 1) ^ (x >> 2)) & 1) and f = 2h + (x >> 2). A row is
// 4.5 bank lines long, so rows of one parity share bank halves. f takes all
// 8 values over the even (and over the odd) rows of any 16-aligned run of 16
// rows (row-fragment reads: 16 rows x one chunk), and h all 4 values over
// the even (odd) rows of rows 0-7, 8-15, {0-3, 8-11} and {4-7, 12-15} of such
// a run (transposed reads: 8 rows x two adjacent chunks, under either
// pairing of 16-lane groups). Both read kinds measure conflict-free on the
// LDS counters; the plainer f = 2 ((row >> 1) & 3) + ((row >> 3) & 1), which
// a 256-byte-pass bank model also finds conflict-free, costs the row-fragment
// reads 4 conflict cycles each.
__device__ __forceinline__ int mla_swz(int row) {
  const int x = (row >> 1) & 7;
  return 2 * ((x & 1) + 2 * (((x >> 1) ^ (x >> 2)) & 1)) + (x >> 2);
}
__device__ __forceinline__ int mla_phys(int c, int row) { return c ^ mla_swz(row); }

// A block's rows [row0, min(row0 + 64, N)) as a buffer resource (reads past
// them return zeros), and copy t (of 72 / W per wave, W waves) of the block
// into an LDS image: 1 KiB per copy, lane l's 16 bytes at dst + 1024 (W t +
// wave) + 16 l.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mla_rsrc(const uint16_t* kvb, int row0, int N) {
  const int rows = __builtin_amdgcn_readfirstlane(min(N - row0, kMlaBN));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(kvb + (size_t)row0 * kMlaDk), (short)0, rows * kMlaRow,
                                           kRsrcWord3);
}
template <int W>
__device__ __forceinline__ void mla_copy_one(__amdgpu_buffer_rsrc_t r, int t, char* dst, int wave, int lane) {
  const int idx = t * W + wave;
  const int pidx = idx * 64 + lane;
  const int row = pidx / 72, pc = pidx % 72;
  cs_dma(r, row * kMlaRow + (mla_phys(pc, row) << 4), dst + idx * 1024);
}
template <int W>
__device__ __forceinline__ void mla_copy_block(const uint16_t* kvb, int row0, int N, char* dst, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = mla_rsrc(kvb, row0, N);
#pragma unroll
  for (int t = 0; t < kMlaCopies / W; ++t) mla_copy_one<W>(r, t, dst, wave, lane);
}

// max and sum over lanes l and l ^ 16 (v_permlane16_swap exchanges the odd
// 16-lane rows of one copy with the even rows of the other)
__device__ __forceinline__ float swap16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Grid: B * (H/16T) * NC workgroups of 128T threads. Chunk c of the key
// blocks as chunk_begin.
template <int T>
__global__ __launch_bounds__(128 * T, 1) void mla_decode_partial(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ KV,
                                                            float* __restrict__ ws_o, float* __restrict__ ws_lse,
                                                            int N, int H, int nc, float c_log2, int q_mode) {
  using S = MlaShape<T>;
  constexpr int W = S::W;
  __shared__ __attribute__((aligned(1024))) char smem[kMlaST * kMlaBlock + S::XCHG];
  const int lane = threadIdx.x & 63, g = lane >> 4, s16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = wave >> 1, half = wave & 1;
  // The H/16T head groups of one (sequence, chunk) take consecutive logical
  // ids, which xcd_remap places on one XCD at once: the groups that fetch a
  // cache block after the first find it in that XCD's L2.
  const int hg = H / S::HEADS;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hgi = L % hg, bc = L / hg;
  const int b = bc / nc, c = bc % nc, h0 = hgi * S::HEADS + 16 * tile;
  const int nblk = (N + kMlaBN - 1) / kMlaBN;
  const int b0 = chunk_begin(c, nblk, nc), b1 = chunk_begin(c + 1, nblk, nc);
  const uint16_t* kvb = KV + (size_t)b * N * kMlaDk;
  const size_t rows = (size_t)(gridDim.x / (hg * nc)) * H;  // B * H
  const size_t row = (size_t)b * H + h0 + s16;               // this lane's head
  float* obase = ws_o + ((size_t)c * rows + (size_t)b * H + h0) * kMlaDv + 256 * half;

  if (b0 == b1) {  // an empty chunk: weight zero in the merge
#pragma unroll
    for (int h = 0; h < 16; ++h) *(f32x4*)(obase + (size_t)h * kMlaDv + 4 * lane) = f32x4{};
    if (half == 0 && g == 0) ws_lse[(size_t)c * rows + row] = -INFINITY;
    return;
  }
  char* xbase = smem + kMlaST * kMlaBlock;
  char* xp_mine = xbase + wave * kMlaXP + lane * 16;
  const char* xp_other = xbase + (wave ^ 1) * kMlaXP + lane * 16;
  float* xf_mine = (float*)(xbase + W * kMlaXP) + wave * 64 + lane;
  const float* xf_other = (const float*)(xbase + W * kMlaXP) + (wave ^ 1) * 64 + lane;
  // row fragments (K and Q): row 16m + s16, chunk 4kk + g at
  // 128 (kk >> 1) + 16 ((4 (kk & 1) + g) ^ f(s16))
  const int fk = mla_swz(s16);
  const int kq[2] = {s16 * kMlaRow + 16 * (g ^ fk), s16 * kMlaRow + 16 * ((4 + g) ^ fk)};
  // transposed reads of dim tile t (dims 256 half + 16t ..): lane s16 of group
  // g addresses row 4g + (s16 >> 2) (+16 for the second read) at dims
  // 16t + 4 (s16 & 3): chunk 32 half + 8 (t >> 2) + ((2 (t & 3) + ((s16 >> 1) & 1)) ^ f(row))
  const int r1 = 4 * g + (s16 >> 2), f1 = mla_swz(r1);
  int vo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    vo[u] = r1 * kMlaRow + 512 * half + 16 * ((2 * u + ((s16 >> 1) & 1)) ^ f1) + 8 * (s16 & 1);
  const int vrow_mine = 32 * half * kMlaRow, vrow_other = 32 * (half ^ 1) * kMlaRow;

  f32x4 o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  // The workgroup's Q rows (16T heads, contiguous) go to ring slot 1 as a
  // 16T-row block (same layout) while block b0 goes to slot 0. Each iteration then
  // issues the copies of the next block (past the chunk end: a duplicate of
  // its last block). There is no L2 prefetch of the block after: a
  // one-read-per-line touch of it, which paid off with four waves per
  // workgroup, slows this kernel down.
  mla_copy_block<W>(Q + ((size_t)b * H + hgi * S::HEADS) * kMlaDk, 0, S::HEADS, smem + kMlaBlock, wave, lane);
  mla_copy_block<W>(kvb, b0 * kMlaBN, N, smem, wave, lane);
  wait_vmcnt<S::CPW>();  // the Q copies, issued first, have landed
  block_barrier();
  // Q^T fragments (B operand): lane holds q[head h0 + s16][32 kk + 8g .. +7],
  // row 16 tile + s16 of the Q image; slot 1 is refilled only after the
  // barrier at the top of the first block
  bf16x8 qf[1][kMlaK];
  {
    const char* qimg = smem + kMlaBlock + 16 * tile * kMlaRow;
#pragma unroll
    for (int kk = 0; kk < kMlaK; ++kk) {
      u32x4 raw = *(LDS_AS const u32x4*)(qimg + kq[kk & 1] + 128 * (kk >> 1));
      raw = apply_q_mode(raw, q_mode);
      qf[0][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  for (int j = b0; j < b1; ++j) {
    const int slot = (j - b0) & 1;
    wait_vmcnt<0>();
    block_barrier();
    // the next block's 9 copies are spread over this block's MFMA streams: 7
    // in the S stream (one per 5 MFMAs), the last 2 early in the PV stream, so
    // that they have most of a block to land
    const __amdgpu_buffer_rsrc_t rnext = mla_rsrc(kvb, min(j + 1, b1 - 1) * kMlaBN, N);
    char* cdst = smem + (slot ^ 1) * kMlaBlock;
    const char* Vs = smem + slot * kMlaBlock;
    const char* Ks = Vs + vrow_mine;
    const int kv0 = j * kMlaBN + 32 * half;
    f32x4 s[2];
    if (kv0 < N) {  // wave-uniform: the second half of the last block may hold no key
      // step i = 2 kk + m: S tile m (keys 16m ..) += K(rows 16m.., k 32kk..) Q^T
      s[0] = f32x4{};
      s[1] = f32x4{};
      auto kread = [&](int i) {
        return *(LDS_AS const bf16x8*)(Ks + (i & 1) * 16 * kMlaRow + kq[(i >> 1) & 1] + 128 * (i >> 2));
      };
      bf16x8 kf[kMlaPfQK];
#pragma unroll
      for (int i = 0; i < kMlaPfQK; ++i) kf[i] = kread(i);
#pragma unroll
      for (int i = 0; i < 2 * kMlaK; ++i) {
        s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[i % kMlaPfQK], qf[0][i >> 1], s[i & 1], 0, 0, 0);
        if (i + kMlaPfQK < 2 * kMlaK) kf[i % kMlaPfQK] = kread(i + kMlaPfQK);
        if (S::s_copy(i) >= 0) mla_copy_one<W>(rnext, S::s_copy(i), cdst, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kv0 + 32 > N) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[m][i] = (kv0 + 16 * m + 4 * g + i >= N) ? -INFINITY : s[m][i];
      }
    } else {
#pragma unroll
      for (int t = 0; t < S::SC; ++t) mla_copy_one<W>(rnext, t, cdst, wave, lane);
#pragma unroll
      for (int m = 0; m < 2; ++m) s[m] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // the block max of each head over both halves (exact), then the common
    // running max; c > 0, so fl(max(s) c) = max(fl(s c))
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    mx = fmaxf(fmaxf(mx, s[0][3]), s[1][0]);
    mx = fmaxf(fmaxf(mx, s[1][1]), s[1][2]);
    mx = swap32_max(swap16_max(fmaxf(mx, s[1][3])));
    *xf_mine = mx;
    block_barrier();
    const float m_new = fmaxf(m_run, fmaxf(mx, *xf_other) * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float p[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[m][i], c_log2, -m_new));
    l_run = __builtin_fmaf(l_run, alpha, ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                                             ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
    bf16x8 pt[2];
    pt[0] = __builtin_convertvector((f32x8{p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]}),
                                    bf16x8);
    *(LDS_AS bf16x8*)(xp_mine) = pt[0];
    block_barrier();
    // P^T of this wave's key half, then of the partner's: own half first, so
    // that the partner's read has landed by the time it is needed
    pt[1] = *(LDS_AS const bf16x8*)(xp_other);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] *= alpha;
    }
    // PV step i = 16 kt + t: O^T tile t += V^T(key half kt) P^T(kt); the
    // transposed reads run kMlaPfPV steps ahead
    auto tr_read = [&](int i, i16x4& a0, i16x4& a1) {
      const int kt = i >> 4, t = i & 15;
      const char* base = Vs + (kt ? vrow_other : vrow_mine) + 128 * (t >> 2) + vo[t & 3];
      a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base));
      a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + 16 * kMlaRow));
    };
    i16x4 va[kMlaPfPV][2];
#pragma unroll
    for (int i = 0; i < kMlaPfPV; ++i) tr_read(i, va[i][0], va[i][1]);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[i % kMlaPfPV][0], va[i % kMlaPfPV][1], 0, 1, 2, 3, 4,
                                                             5, 6, 7));
      o[i & 15] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pt[i >> 4], o[i & 15], 0, 0, 0);
      if (i + kMlaPfPV < 32) tr_read(i + kMlaPfPV, va[i % kMlaPfPV][0], va[i % kMlaPfPV][1]);
      if (S::pv_copy(i) >= 0) mla_copy_one<W>(rnext, S::pv_copy(i), cdst, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  // the row sum: this wave's keys (over its four lane groups), then the
  // partner's (same alpha sequence)
  const float l_mine = swap32_sum(swap16_sum(l_run));
  block_barrier();  // the partner has read this wave's last max; every wave is done with the ring
  *xf_mine = l_mine;
  block_barrier();
  const float l_tot = l_mine + *xf_other;
  const float inv = 1.0f / l_tot;
  // O^T (lane = head, registers = dims) goes through LDS so that each store
  // writes one head's 256 dims (1 KiB) contiguously: [head][dim] per wave,
  // 16-byte chunk k of head h at k ^ h (conflict-free both ways)
  char* st = smem + wave * (16 * 1024);
#pragma unroll
  for (int t = 0; t < 16; ++t) *(LDS_AS f32x4*)(st + s16 * 1024 + (((4 * t + g) ^ s16) << 4)) = o[t] * inv;
  // (a wave reads back only its own rows; its LDS accesses complete in order)
#pragma unroll 4
  for (int h = 0; h < 16; ++h)
    *(f32x4*)(obase + (size_t)h * kMlaDv + 4 * lane) = *(LDS_AS const f32x4*)(st + h * 1024 + ((lane ^ h) << 4));
  if (half == 0 && g == 0) ws_lse[(size_t)c * rows + row] = kLn2 * (m_run + __builtin_amdgcn_logf(l_tot));
}

// Merge of the NC chunk partials of one (b, h) row, for NC <= kMlaMergePF
// (many rows, few chunks): one wave per row, four rows per workgroup, lane l
// owning output dims 8l .. 8l + 7. Every lane reads all NC chunk LSEs (the
// same addresses in every lane: one request each) and its 8 dims of every
// partial, all issued before any weight is known, so the merge costs one
// memory round trip; no barrier. (Few rows with many chunks go to
// mla_combine_wide instead.) Weights and sums run over the chunks in order:
// w_c = exp(LSE_c - max), O = sum w_c O_c / sum w_c, LSE = max + ln(sum w_c)
// (an empty chunk has LSE -inf and weight 0).
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
__global__ __launch_bounds__(256, 1) void mla_combine_wide(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_lse,
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


// MLA decoding: H a multiple of 64 (64 heads per workgroup, or 16 when that
// leaves CUs idle); chunks sized so
// that one resident round of workgroups (one per CU) covers the cache, at
// least two 64-row blocks per chunk (one-block chunks: B = 1 took 24.7
// against 20.6 us, the per-workgroup Q load and partial stores then
// dominate).
struct MlaPlan {
  int nc, tiles;  // key chunks; 16-head tiles per workgroup (4 or 1)
  long long groups, rows;
  size_t ws_bytes;  // nc * rows * (Dv + 1) floats
};

int mla_plan(int B, int H, int N, MlaPlan* p) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (H % 64 != 0) return ATTN_ERR_BAD_SHAPE;
  p->rows = (long long)B * H;
  p->groups = (long long)B * (H / 64);
  p->tiles = 4;
  p->nc = 0;
  p->ws_bytes = 0;
  if (p->rows == 0) return ATTN_OK;
  if (N < 1) return ATTN_ERR_BAD_SHAPE;
  long long elems = 0;
  if (__builtin_mul_overflow((long long)B * N, (long long)kMlaDk, &elems) || elems > (1LL << 50) ||
      p->rows > INT_MAX)
    return ATTN_ERR_BAD_SHAPE;
  const long long nblk = (N + kMlaBN - 1) / kMlaBN;
  auto chunks = [nblk](long long groups) {
    long long n = (256 + groups - 1) / groups;  // one resident round (one workgroup per CU)
    n = std::min(n, std::max(1LL, nblk / 2));   // at least two blocks per chunk
    return std::min(n, (long long)kDecodeMaxChunks);
  };
  long long nc = chunks(p->groups);
  if (p->groups * nc < 256) {  // 64-head workgroups would leave CUs idle: 16-head ones
    p->tiles = 1;
    p->groups = (long long)B * (H / 16);
    nc = chunks(p->groups);
  }
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
  const dim3 grid((unsigned)(p.groups * p.nc));
  if (p.tiles == 4)
    hipLaunchKernelGGL(mla_decode_partial<4>, grid, dim3(512), 0, (hipStream_t)stream, (const uint16_t*)q,
                       (const uint16_t*)kv, ws_o, ws_lse, N, H, p.nc, scale_args(scale).c_log2,
                       scale_args(scale).q_mode);
  else
    hipLaunchKernelGGL(mla_decode_partial<1>, grid, dim3(128), 0, (hipStream_t)stream, (const uint16_t*)q,
                       (const uint16_t*)kv, ws_o, ws_lse, N, H, p.nc, scale_args(scale).c_log2,
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
