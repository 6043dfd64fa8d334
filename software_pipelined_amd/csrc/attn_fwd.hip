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
// wgmma ping-pong are prior art):
//   * one workgroup = NW wavefronts x 32 query rows (BM = 32*NW), one SIMD
//     pair per two waves; each wave owns its 32 queries end to end;
//   * S is formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K (from LDS) is the A operand and Q^T (kept in VGPRs for the whole
//     loop) is the B operand, so each lane's accumulator column is one query
//     and row max / row sum reduce within the lane plus one lane^32 swap
//     (v_permlane32_swap);
//   * O^T += V^T P^T with the same instruction: P^T goes straight from the
//     S accumulators into the B operand (cvt to bf16, no LDS round trip),
//     V^T is read with the gfx950 transposing LDS read ds_read_b64_tr_b16;
//   * K/V blocks are double-buffered in LDS and filled with
//     global_load_lds_dwordx4 (HBM -> LDS without VGPRs), one block ahead of
//     the block being computed; the destination layout is XOR-swizzled per
//     row by choosing which global chunk each lane fetches;
//   * exp2 runs on v_exp_f32 with scale*log2(e) folded into one FMA;
//   * the O *= alpha rescale is skipped by a whole wave when none of its 32
//     rows raised its running max in the block (alpha == 1 exactly). The max
//     itself is tracked exactly, never lazily: a stale max makes the
//     dominant key's weight 2^delta instead of exactly 1, and its bf16
//     rounding then costs up to 2^-9 |v| on near-one-hot rows;
//   * workgroup ids are remapped so that consecutive query tiles of one head
//     run on one XCD (shared L2 for that head's K/V); causal grids start with
//     the heaviest tiles.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, int NW, int BN>
struct Tile {
  static constexpr int BM = 32 * NW;                 // query rows per workgroup
  static constexpr int RC = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int MAT_BYTES = BN * D * 2;       // one K (or V) block in LDS
  static constexpr int STAGE_BYTES = 2 * MAT_BYTES;  // K + V
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;  // two stages
  static constexpr int LOADS = MAT_BYTES / (16 * 64 * NW);  // 1 KiB wave loads per matrix
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BN % 32 == 0, "BN multiple of 32");
  static_assert(LOADS * 16 * 64 * NW == MAT_BYTES, "block must split evenly over waves");
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

// Issue the HBM -> LDS copy of BN rows (starting at row0) of one [N][D]
// matrix. Every wave moves LOADS x 1 KiB; lane l's 16 bytes land at
// dst + 16*l, so the swizzle is applied by choosing the source chunk.
// Rows past N are clamped to row N-1 (finite data; those keys are masked).
template <int D, int NW, int BN, bool IS_V>
__device__ __forceinline__ void issue_block_load(const uint16_t* __restrict__ src, int row0, int N,
                                                 char* dst, int wave, int lane) {
  using T = Tile<D, NW, BN>;
#pragma unroll
  for (int t = 0; t < T::LOADS; ++t) {
    const int slot0 = (t * NW + wave) * 64;
    const int p = slot0 + lane;
    const int row = p / T::RC;
    const int pc = p % T::RC;
    const int c = pc ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
    const int grow = min(row0 + row, N - 1);
    const uint16_t* g = src + (size_t)grow * D + c * 8;
    __builtin_amdgcn_global_load_lds((GLB_AS void*)g, (LDS_AS void*)(dst + slot0 * 16), 16, 0, 0);
  }
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

template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c_log2, int negate_q) {
  using T = Tile<D, NW, BN>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;  // which half of the wave
  const int lq = lane & 31;  // query column owned by this lane

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qtiles;
  const int tq = L % n_qtiles;
  const int tile = CAUSAL ? (n_qtiles - 1 - tq) : tq;
  const int q0 = tile * T::BM;
  const int q0w = q0 + wave * 32;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // KV range of the workgroup and of this wave.
  const int kv_end_wg = CAUSAL ? min(N, q0 + T::BM) : N;
  const int kv_end_w = CAUSAL ? min(N, q0w + 32) : N;
  const int nblk = (kv_end_wg + BN - 1) / BN;

  // Prefetch block 0 before touching Q so the copies overlap the Q load.
  issue_block_load<D, NW, BN, false>(Kh, 0, N, smem, wave, lane);
  issue_block_load<D, NW, BN, true>(Vh, 0, N, smem + T::MAT_BYTES, wave, lane);

  // Q^T as MFMA B operand: lane holds Q[q][kk*16 + h*8 .. +7] for its query q.
  bf16x8 qf[D / 16];
  {
    const int qrow = min(q0w + lq, N - 1);
    const uint16_t* qp = Qh + (size_t)qrow * D + h * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 raw = *(const u32x4*)(qp + kk * 16);
      if (negate_q) raw ^= 0x80008000u;  // exact sign flip of 8 bf16 values
      qf[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits, log2 units
  float l_run = 0.f;        // this lane's half of the running row sum

  const int qi = q0w + lq;  // this lane's query index (may be >= N in a ragged tile)

  for (int j = 0; j < nblk; ++j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < nblk) {
      char* st = smem + ((j + 1) & 1) * T::STAGE_BYTES;
      issue_block_load<D, NW, BN, false>(Kh, (j + 1) * BN, N, st, wave, lane);
      issue_block_load<D, NW, BN, true>(Vh, (j + 1) * BN, N, st + T::MAT_BYTES, wave, lane);
    }
    const int kv0 = j * BN;
    if (kv0 >= kv_end_w) continue;  // wave-uniform: block entirely masked for this wave

    const char* Ks = smem + (j & 1) * T::STAGE_BYTES;
    const char* Vs = Ks + T::MAT_BYTES;

    // ---- mma_qk: S^T[key][query] for BN keys, 32 keys per accumulator tile
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = f32x16{};
      const int row = kb * 32 + lq;
      const char* rbase = Ks + row * (D * 2);
      const int sw = swz_k<D>(row);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int ch = (2 * kk + h) ^ sw;
        bf16x8 a = *(LDS_AS const bf16x8*)(rbase + ch * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }

    // ---- mask (only blocks that straddle the diagonal or the end of K)
    const bool need_mask = (kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const bool dead = (key >= N) || (CAUSAL && key > qi);
          s[kb][r] = dead ? -INFINITY : s[kb][r];
        }
    }

    // ---- online softmax
    float bmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) bmax = fmaxf(bmax, fmaxf(s[kb][r], s[kb][r + 1]));
    bmax = swap32_max(bmax);
    const float mb = bmax * c_log2;
    const float m_new = fmaxf(m_run, mb);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 if unchanged, 0 at start
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_new));
        s[kb][r] = p;
        psum += p;
      }
    l_run = __builtin_fmaf(l_run, alpha, psum);

    // ---- rescale (skipped by the whole wave when no row moved its max)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) o[t] *= alpha;
    }

    // ---- mma_pv: O^T[dim][query] += V^T[dim][key] P^T[key][query]
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // B operand: 8 keys of this lane's half, taken from accumulator
        // registers 8*hf .. 8*hf+7 (keys kb*32 + 16*hf + {0..3, 8..11} + 4*h).
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[kb][8 * hf + e];
        const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
        // A operand rows: the same 8 keys, read transposed from V.
        const int kbase0 = kb * 32 + 16 * hf + 4 * h;
        const int ci = lane & 15;
        const int g2 = (lane >> 4) & 1;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int dd = t * 32 + g2 * 16 + 4 * (ci & 3);
          const int chunk = dd >> 3;
          const int within = (dd & 7) * 2;
          const int r0 = kbase0 + (ci >> 2);
          const int r1 = r0 + 8;
          const char* a0 = Vs + r0 * (D * 2) + ((chunk ^ swz_v<D>(r0)) * 16) + within;
          const char* a1 = Vs + r1 * (D * 2) + ((chunk ^ swz_v<D>(r1)) * 16) + within;
          i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
          i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a1);
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[t], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: normalise, write O and LSE
  const float l_tot = swap32_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qi < N) {
    float* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {o[t][4 * g] * inv, o[t][4 * g + 1] * inv, o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv};
        *(f32x4*)(orow + t * 32 + g * 8 + h * 4) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + qi] = kLn2 * (m_run + __builtin_amdgcn_logf(l_tot));
  }
}

// ---------------------------------------------------------------- host side

typedef hipError_t (*launch_fn)(const void*, const void*, const void*, float*, float*, int, int,
                                int, int, float, hipStream_t);

template <int D, int NW, int BN>
hipError_t launch(const void* q, const void* k, const void* v, float* out, float* lse, int B,
                  int H, int N, int causal, float scale, hipStream_t stream) {
  using T = Tile<D, NW, BN>;
  const int n_qt = (N + T::BM - 1) / T::BM;
  const long long G = (long long)B * H * n_qt;
  const float c = fabsf(scale) * kLog2e;
  const int neg = scale < 0.f;
  if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, BN, true>), dim3((unsigned)G), dim3(NW * 64), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, out,
                       lse, N, n_qt, c, neg);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, BN, false>), dim3((unsigned)G), dim3(NW * 64), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, out,
                       lse, N, n_qt, c, neg);
  return hipGetLastError();
}

struct Variant {
  const char* name;
  int d, bm, bn, waves, lds;
  launch_fn fn;
};

#define VARIANT(NAME, D, NW, BN) \
  Variant { NAME, D, 32 * NW, BN, NW, Tile<D, NW, BN>::LDS_BYTES, &launch<D, NW, BN> }

const Variant kVariants[] = {
    VARIANT("d64_bm256_bn64_w8", 64, 8, 64),     // 0
    VARIANT("d128_bm256_bn64_w8", 128, 8, 64),   // 1
    VARIANT("d256_bm128_bn64_w4", 256, 4, 64),   // 2
    VARIANT("d64_bm128_bn64_w4", 64, 4, 64),     // 3
    VARIANT("d128_bm128_bn64_w4", 128, 4, 64),   // 4
    VARIANT("d64_bm256_bn128_w8", 64, 8, 128),   // 5
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int default_variant(int d, int causal) {
  (void)causal;
  switch (d) {
    case 64: return 0;
    case 128: return 1;
    case 256: return 2;
    default: return -1;
  }
}

int validate(const void* q, const void* k, const void* v, const float* out, const float* lse,
             int B, int H, int N, int d, float scale, int bm) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale) || scale == 0.f) return ATTN_ERR_BAD_SCALE;
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

}  // extern "C"
