// attn_decode.hip -- split-KV decoding (attn_fwd_decode) on MI355X (gfx950).
//
// Part of libattn.so; the C ABI is declared in include/attn.h.

#include <mutex>

#include "attn_common.h"

namespace {

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

// As cs_dma, with the non-temporal cache policy: every K/V line is read once
// per call, so it is streamed rather than kept in L2 (B = 32: 328 against
// 361 us per call, B = 1: 17.6 against 19.7 us).
__device__ __forceinline__ void cs_dma_stream(__amdgpu_buffer_rsrc_t r, int voff, char* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(LDS_AS void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r), "s"(m0)
               : "m0", "memory");
}

// HBM -> LDS copy t of a wave-private block (inline assembly, as cs_dma, so
// the compiler's conservative wait before the transposing V reads does not
// drain the next block's copy; the copies are waited for with wait_vmcnt).
template <int D, int BN, bool IS_V>
__device__ __forceinline__ void issue_copy_wave(const uint16_t* __restrict__ src, int row0, int N, char* dst,
                                                int lane, int t) {
  cs_dma_stream(block_rsrc<D, BN>(src, row0, N), (int)block_lane_offset<D, 1, BN, IS_V>(t, 0, lane),
                dst + t * 64 * 16);
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


// Ring slots per wave: three at d = 128 (two blocks in flight behind the one
// being multiplied, three waves per CU: 1-6 % faster than two slots and four
// waves once the copies stream), two otherwise (at d = 256 three slots would
// leave one wave per CU).
constexpr int decode_slots(int d) { return d == 128 ? 3 : 2; }

// Grid: (B*H*n_qt) x (NC / NW) workgroups of NW waves; wave w of workgroup
// (x, y) takes chunk y*NW + w of query tile x % n_qt of head x / n_qt.
template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void attn_decode_partial(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int BH, int Nq, int Nkv, int n_qt, int nc,
    float c_log2, int q_mode) {
  constexpr int ST = decode_slots(D);
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
  load_q<D, 1>(Q + (size_t)bh * Nq * D, qt0, Nq, q_mode, qf, lane);
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
  // blocks b0 .. b0 + ST - 2 go out first; iteration j refills the slot of
  // block j - 1 with block j + ST - 1 and waits for block j only
#pragma unroll
  for (int i = 0; i < ST - 1; ++i)
    if (b0 + i < b1) copy_block_wave<D, BN>(Kh, Vh, (b0 + i) * BN, Nkv, ks(i), vs(i), lane);
  for (int j = b0; j < b1; ++j) {
    const int slot = (j - b0) % ST;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the slot about to be refilled are done
    if (j + ST - 1 < b1) {
      const int ns = (j + ST - 1 - b0) % ST;
      copy_block_wave<D, BN>(Kh, Vh, (j + ST - 1) * BN, Nkv, ks(ns), vs(ns), lane);
      wait_vmcnt<(ST - 1) * PER_BLOCK>();  // block j has landed, the later ones may stay in flight
    } else if (ST == 3 && j + 1 < b1) {
      wait_vmcnt<PER_BLOCK>();
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
// holds its first partials in registers. A thread owns four consecutive
// output dimensions (16-byte loads) of one slice of the chunks: S = 1024 / D
// slices, chunks c = slice + i S; the first 128 chunks of a row are loaded
// before any weight is known, so up to 128 chunks cost one memory round
// trip. The slices are added in LDS in a fixed order (deterministic).

template <int D>
__global__ __launch_bounds__(256, 1) void attn_decode_combine(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_lse,
                                                             float* __restrict__ O, float* __restrict__ LSE,
                                                             int rows, int nc) {
  constexpr int DG = D / 4;       // threads per slice (four dims each)
  constexpr int S = 256 / DG;     // chunk slices: 16 at d = 64, 8 at d = 128, 4 at d = 256
  constexpr int PF = 128 / S;     // partials per thread loaded before the weights are known
  __shared__ float w_sh[kDecodeMaxChunks];
  __shared__ f32x4 red4[S][DG];
  __shared__ float red[8];
  const int tid = threadIdx.x, row = blockIdx.x;
  const int g = tid % DG, sl = tid / DG;
  const float* base = ws_o + (size_t)row * D + 4 * g;  // chunk c at base + c * rows * D
  const size_t cstride = (size_t)rows * D;
  f32x4 pre[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int c = sl + i * S;
    pre[i] = c < nc ? *(const f32x4*)(base + (size_t)c * cstride) : f32x4{};
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
  f32x4 acc = {};
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int c = sl + i * S;
    if (c < nc) acc += w_sh[c] * pre[i];
  }
  int c = sl + PF * S;
  for (; c + 3 * S < nc; c += 4 * S) {
    const float* src = base + (size_t)c * cstride;
    const size_t st = (size_t)S * cstride;
    const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + st), d2 = *(const f32x4*)(src + 2 * st),
                e = *(const f32x4*)(src + 3 * st);
    acc += w_sh[c] * a;
    acc += w_sh[c + S] * b;
    acc += w_sh[c + 2 * S] * d2;
    acc += w_sh[c + 3 * S] * e;
  }
  for (; c < nc; c += S) acc += w_sh[c] * *(const f32x4*)(base + (size_t)c * cstride);
  red4[sl][g] = acc;
  __syncthreads();
  if (tid < DG) {
    f32x4 o = red4[0][tid];
#pragma unroll
    for (int k = 1; k < S; ++k) o += red4[k][tid];
    *(f32x4*)(O + (size_t)row * D + 4 * tid) = o / wsum;
  }
  if (tid == 0) LSE[row] = mx + kLn2 * __builtin_amdgcn_logf(wsum);
}

// Split-KV decoding: 32-key blocks, 4 waves per workgroup at d = 64, 3 at
// d = 128 and 2 at d = 256 (whose 64 KiB ring per wave fills the LDS). Each
// wave's K/V ring holds decode_slots(d) slots x 2 matrices x 32 keys x d
// bf16, so the 160 KiB LDS of a CU keeps 8 waves resident at d = 64, 3 at
// d = 128 and 2 at d = 256; the chunks are sized so that one resident round
// of waves (256 CUs) streams the cache, rounded up to a multiple of the waves
// per workgroup.
constexpr int kDecodeBN = 32;
constexpr int kDecodeCUs = 256;
constexpr int kDecodeLdsPerCU = 160 * 1024;

constexpr int decode_waves(int d, int nw) {
  return kDecodeCUs * (kDecodeLdsPerCU / (nw * decode_slots(d) * 2 * kDecodeBN * d * 2)) * nw;
}
static_assert(decode_waves(64, 4) == 2048 && decode_waves(128, 3) == 768 && decode_waves(256, 2) == 512,
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
  p->nw = d == 256 ? 2 : (d == 128 ? 3 : 4);
  p->n_qt = (Nq + 31) / 32;
  p->nc = 0;
  p->ws_bytes = 0;
  if (rows == 0) return ATTN_OK;
  if (Nkv < 1) return ATTN_ERR_BAD_SHAPE;  // a query with no key has no softmax
  const long long groups = bh * p->n_qt;
  if (elems_q > (1LL << 50) || elems_kv > (1LL << 50) || !grid_fits(groups, 256) || !grid_fits(rows, 256))
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
  const ScaleArgs sa = scale_args(scale);
  const float c = sa.c_log2;
  const int neg = sa.q_mode;
  clear_last_hip_error();
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

// ---------------------------------------------------------------- no-allocation entry
// attn_fwd_decode_static keeps the chunk partials in this fixed device array
// instead of a caller workspace, for callers that cannot allocate. Each GPU
// the library runs on holds its own copy until the process ends. In host
// code the array's name is not a device address: the address of the current
// device's copy comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of scratch (looked up on its first use).
int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

// Argument checks shared by both decoding entries (before any HIP call).
int decode_check(const DecodePlan& p, const void* q, const void* k, const void* v, const float* out,
                 const float* lse, float scale) {
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_BAD_SCALE;  // NaN or +-Inf
  if (p.rows == 0) return ATTN_OK;
  if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

hipError_t launch_decode_d(int d, const DecodePlan& p, const void* q, const void* k, const void* v, float* out,
                           float* lse, int BH, int Nq, int Nkv, float scale, void* ws, hipStream_t stream) {
  switch (d) {
    case 64: return launch_decode<64, 4>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, ws, stream);
    case 128: return launch_decode<128, 3>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, ws, stream);
    default: return launch_decode<256, 2>(p, q, k, v, out, lse, BH, Nq, Nkv, scale, ws, stream);
  }
}

}  // namespace

extern "C" {

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
  st = decode_check(p, q, k, v, out, lse, scale);
  if (st != ATTN_OK || p.rows == 0) return st;
  if (!workspace) return ATTN_ERR_NULL_PTR;
  if (((uintptr_t)workspace & 15) != 0) return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < p.ws_bytes) return ATTN_ERR_WORKSPACE;
  const hipError_t e = launch_decode_d(d, p, q, k, v, out, lse, B * H, Nq, Nkv, scale, workspace,
                                       (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_decode_static_max_bytes(void) { return kDecodeScratchBytes; }

int attn_fwd_decode_static(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
                           int Nq, int Nkv, int d, float scale, void* stream) {
  DecodePlan p;
  int st = decode_plan(B, H, Nq, Nkv, d, &p);
  if (st != ATTN_OK) return st;
  st = decode_check(p, q, k, v, out, lse, scale);
  if (st != ATTN_OK || p.rows == 0) return st;
  if (p.ws_bytes > kDecodeScratchBytes) return ATTN_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != ATTN_OK) return st;
  const hipError_t e = launch_decode_d(d, p, q, k, v, out, lse, B * H, Nq, Nkv, scale, ws, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
