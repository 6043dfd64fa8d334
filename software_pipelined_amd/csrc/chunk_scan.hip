// chunk_scan.hip -- Mamba2 ChunkScan (chunk_scan) on MI355X (gfx950).
//
// Part of libattn.so; the C ABI is declared in include/attn.h.

#include "attn_common.h"

namespace {

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
// this one is computed. Logical workgroup ids run over heads fastest and
// stay on one XCD in runs (xcd_remap), so the heads sharing one cb chunk run
// together on one L2.
constexpr int kCsP = 64;   // channels per head
constexpr int kCsBK = 32;  // steps per block
// One ring slot: the x block (32 x 64 bf16, V layout), the cb columns of the
// block for the workgroup's rows (64 bytes per row, 16-byte chunks XORed with
// (row >> 1) & 3), then dt and dA_cumsum of the block's 32 steps (128 bytes
// each, copied by 8 lanes).
constexpr int kCsX = kCsBK * kCsP * 2;
template <int RW>
struct CsSlot {
  static constexpr int CB = RW * kCsBK * 2;    // cb columns of the block for the workgroup's RW rows
  static constexpr int BYTES = kCsX + CB + 2 * 128;
};


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
    if (lane < 8) {  // 128 bytes each: the other lanes would only write zeros
      cs_dma(rd, lane * 16, slot + kCsX + CsSlot<RW>::CB);
      cs_dma(ra, lane * 16, slot + kCsX + CsSlot<RW>::CB + 128);
    }
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
  // the ring, reused at the end to stage each wave's 32 output rows
  __shared__ __attribute__((aligned(1024))) char smem[std::max(2 * SLOT, NW * 32 * kCsP * 4)];
  static_assert(QT == 1, "one staged 32-row image per wave");
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nparts = (L + RW - 1) / RW;
  // logical id: heads fastest, then parts, chunks, sequences; xcd_remap keeps
  // consecutive ids on one XCD, so the heads (and parts) of one chunk share
  // that XCD's L2 copy of the chunk's cb
  const int L_id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L_id % H, part = (L_id / H) % nparts, c = (L_id / (H * nparts)) % nc, b = L_id / (H * nparts * nc);
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
        dav[hf][e] = *(LDS_AS const f32x4*)(dts + 128 + (16 * hf + 8 * e + 4 * hl) * 4);
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
  // Output rows through LDS, so that each store instruction writes four whole
  // 256-byte rows: the accumulators hold, per lane, 4-channel groups of one
  // row. All waves have finished with the ring before it is reused. Row r of
  // a wave's 32 x 64 fp32 image keeps its 16-byte chunk c at c ^ (r & 15),
  // so neither the row-wise writes nor the row-major reads conflict.
  block_barrier();
  char* stage = smem + wave * (32 * kCsP * 4);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = lane & 31;
#pragma unroll
    for (int t = 0; t < kCsP / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = (t * 32 + g * 8 + hl * 4) / 4;  // 16-byte chunk of the row
        *(LDS_AS f32x4*)(stage + r * (kCsP * 4) + ((c ^ (r & 15)) << 4)) =
            f32x4{o[qt][t][4 * g], o[qt][t][4 * g + 1], o[qt][t][4 * g + 2], o[qt][t][4 * g + 3]};
      }
    // the rows are read back by other lanes of the same wave: its LDS
    // accesses complete in order; the fence keeps the compiler from moving
    // the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int c = lane & 15;
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 4 * i + (lane >> 4);
      v[i] = *(LDS_AS const f32x4*)(stage + rr * (kCsP * 4) + ((c ^ (rr & 15)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = mw + 32 * qt + 4 * i + (lane >> 4);
      if (m < Lc) *(f32x4*)(OUT + (((size_t)b * S + c0 + m) * H + h) * kCsP + 4 * c) = v[i];
    }
  }
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

}  // namespace

extern "C" {

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
  if (!grid_fits(groups * parts, 256)) return ATTN_ERR_BAD_SHAPE;
  clear_last_hip_error();
  hipLaunchKernelGGL((chunk_scan_fwd<4, kCsRows / 128>), dim3((unsigned)(groups * parts)), dim3(256), 0,
                     (hipStream_t)stream,
                     (const uint16_t*)x, (const uint16_t*)cb, dt, dA_cumsum, out, S, H, L, nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
