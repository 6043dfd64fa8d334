// mla_decode.hip -- MLA decoding (mla_decode) on MI355X (gfx950).
//
// Part of libattn.so; the C ABI is declared in include/attn.h.

#include "attn_common.h"

namespace {

// ---------------------------------------------------------------- MLA decoding
// Multi-head latent attention decoding in the absorbed form (the decoding
// operator the PipeThreader summary page's "Discussion" paragraph cites,
// written there in about 80 lines against 500-plus by hand): all H query heads of a sequence attend to one shared cache of
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
                                                            int N, int H, int nc, float c_log2, int q_mode) {
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
      raw = apply_q_mode(raw, q_mode);
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
  hipLaunchKernelGGL(mla_decode_partial, dim3((unsigned)p.groups, (unsigned)p.nc), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)kv, ws_o, ws_lse, N, H, p.nc, scale_args(scale).c_log2,
                     scale_args(scale).q_mode);
  hipLaunchKernelGGL(mla_combine, dim3((unsigned)p.rows), dim3(256), 0, (hipStream_t)stream, (const float*)ws_o,
                     (const float*)ws_lse, out, lse, (int)p.rows, p.nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
