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
// One ring slot: the x blocks of the workgroup's HT heads (32 x 64 bf16
// each, V layout), the cb columns of the block for the workgroup's rows (64
// bytes per row, 16-byte chunks XORed with cs_cb_swz(row)), then dt and
// dA_cumsum of the block's 32 steps for each head (128 bytes each, copied by
// 8 lanes).
constexpr int kCsX = kCsBK * kCsP * 2;
// A lane reads 8 bytes (half a chunk) of its row; a read pass serves 32 lanes,
// i.e. 32 rows with the same half, and four rows share one 256-byte bank
// line. XOR with (row >> 1) & 3 leaves a pass 4-way conflicted; (row >> 2) & 3
// would make it 2-way (the least this layout allows) and cut the conflict
// cycles to a third, but measured 2.5 % slower on the whole kernel.
__device__ __forceinline__ int cs_cb_swz(int row) { return (row >> 1) & 3; }
template <int RW, int HT>
struct CsSlot {
  static constexpr int CB = RW * kCsBK * 2;  // cb columns of the block for the workgroup's RW rows
  static constexpr int DT = HT * kCsX + CB;  // dt, dA_cumsum of head hh at DT + 256 hh, DT + 256 hh + 128
  static constexpr int BYTES = DT + HT * 256;
};

// All copies of block j (steps k0 = 32j ..): x rows of the HT heads (rows
// past the chunk read zeros), the cb columns k0 .. k0+31 of the workgroup's
// rows [max(k0, r0), min(L, r0 + RW)) (earlier rows never see the block), dt
// and dA_cumsum of each head.
template <int NW, int RW, int HT>
__device__ __forceinline__ void cs_copy_block(const uint16_t* xh, const uint16_t* cbc, const float* dtc,
                                              const float* dac, size_t head_stride, int j, int Lc, int L, int r0,
                                              int row_stride, char* slot, int wave, int lane) {
  const int k0 = j * kCsBK;
  {  // x: 4 KiB per head, one 1 KiB copy (8 rows of one head) per wave and head
    const int rows_valid = min(kCsBK, Lc - k0);
    const int bytes = __builtin_amdgcn_readfirstlane((rows_valid - 1) * row_stride * 2 + HT * kCsP * 2);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xh + (size_t)k0 * row_stride), (short)0, bytes, kRsrcWord3);
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
      const int pidx = wave * 64 + lane;
      const int row = pidx >> 3, pc = pidx & 7;
      cs_dma(r, row * row_stride * 2 + hh * kCsP * 2 + ((pc ^ swz_v<kCsP>(row)) << 4), slot + hh * kCsX + wave * 1024);
    }
  }
  {  // cb: rows of 64 bytes, 16 per 1 KiB copy, dealt over the waves
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)cbc, (short)0, L * L * 2, kRsrcWord3);
    const int first = max(k0, r0), n = (min(L, r0 + RW) - first) / 16;
    for (int t = wave; t < n; t += NW) {
      const int pidx = t * 64 + lane;
      const int row = first + (pidx >> 2), pc = pidx & 3;
      const int c = pc ^ cs_cb_swz(row);
      cs_dma(r, (row * L + k0) * 2 + (c << 4), slot + HT * kCsX + (first - r0) * 64 + t * 1024);
    }
  }
  if (wave < HT) {  // dt and dA_cumsum of the block's 32 steps, head `wave`
    const size_t ho = (size_t)wave * head_stride + k0;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)(dtc + ho), (short)0, 128, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(dac + ho), (short)0, 128, kRsrcWord3);
    if (lane < 8) {  // 128 bytes each: the other lanes would only write zeros
      cs_dma(rd, lane * 16, slot + CsSlot<RW, HT>::DT + wave * 256);
      cs_dma(ra, lane * 16, slot + CsSlot<RW, HT>::DT + wave * 256 + 128);
    }
  }
}

// A workgroup of NW waves covers RW = 32 NW chunk rows starting at r0 (wave w:
// rows r0 + 32w .. r0 + 32w + 31) for HT consecutive heads; a chunk takes
// ceil(L / RW) workgroups per head group. With HT = 2 the two heads share
// the cb columns (copied and read once per block) and their x rows are
// adjacent in memory.
template <int NW, int HT>
__global__ __launch_bounds__(NW * 64, HT == 2 ? 4 : 5) void chunk_scan_fwd(const uint16_t* __restrict__ X,
                                                                           const uint16_t* __restrict__ CB,
                                                         const float* __restrict__ DT, const float* __restrict__ DAC,
                                                         float* __restrict__ OUT, int S, int H, int L, int nc) {
  static_assert(NW == 4, "one 1 KiB copy per wave covers a quarter of a 32 x 64 bf16 block");
  static_assert(HT <= NW, "the dt / dA_cumsum copies take one wave per head");
  constexpr int RW = 32 * NW;
  constexpr int SLOT = CsSlot<RW, HT>::BYTES;
  // the ring, reused at the end to stage each wave's 32 output rows
  __shared__ __attribute__((aligned(1024))) char smem[std::max(2 * SLOT, NW * 32 * kCsP * 4)];
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nparts = (L + RW - 1) / RW;
  const int HG = H / HT;  // head groups
  // logical id: head groups fastest, then parts, chunks, sequences;
  // xcd_remap keeps consecutive ids on one XCD, so the heads (and parts) of
  // one chunk share that XCD's L2 copy of the chunk's cb
  const int L_id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = (L_id % HG) * HT, part = (L_id / HG) % nparts, c = (L_id / (HG * nparts)) % nc,
            b = L_id / (HG * nparts * nc);
  const int c0 = c * L, Lc = min(L, S - c0), r0 = part * RW;
  if (r0 >= Lc) return;  // workgroup-uniform: this part of a short last chunk is empty
  const int nblk = (min(Lc, r0 + RW) + kCsBK - 1) / kCsBK;
  const int row_stride = H * kCsP;
  const uint16_t* xh = X + ((size_t)b * S + c0) * row_stride + (size_t)h * kCsP;
  const uint16_t* cbc = CB + ((size_t)b * nc + c) * L * L;
  const size_t head_stride = (size_t)nc * L;  // dt / dA_cumsum of the next head
  const size_t sc = (((size_t)b * H + h) * nc + c) * L;
  const float* dtc = DT + sc;
  const float* dac = DAC + sc;
  const int mw = r0 + 32 * wave;  // first chunk row of this wave
  const int m = mw + (lane & 31);  // this lane's row

  float dam[HT];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) dam[hh] = dac[hh * head_stride + min(m, Lc - 1)];
  const LdsOffsets<kCsP> off(lane);
  f32x16 o[HT][1][kCsP / 32];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int t = 0; t < kCsP / 32; ++t) o[hh][0][t] = f32x16{};

  cs_copy_block<NW, RW, HT>(xh, cbc, dtc, dac, head_stride, 0, Lc, L, r0, row_stride, smem, wave, lane);
  for (int j = 0; j < nblk; ++j) {
    wait_vmcnt<0>();
    block_barrier();
    if (j + 1 < nblk)
      cs_copy_block<NW, RW, HT>(xh, cbc, dtc, dac, head_stride, j + 1, Lc, L, r0, row_stride,
                                smem + ((j + 1) & 1) * SLOT, wave, lane);
    const int k0 = j * kCsBK;
    if (mw >= Lc || k0 > mw + 31) continue;  // wave-uniform: no row of this wave sees the block
    const char* slot = smem + (j & 1) * SLOT;
    // this lane's cb values: row m, steps k0 + 16hf + 8e + 4hl + i (rows below
    // k0 hold stale data; their terms are masked)
    const char* cbr = slot + HT * kCsX + (m - r0) * 64 + 8 * hl;
    const int sw = cs_cb_swz(m);
    u32x2 raw[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 2; ++e) raw[hf][e] = *(LDS_AS const u32x2*)(cbr + (((2 * hf + e) ^ sw) << 4));
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
      const char* dts = slot + CsSlot<RW, HT>::DT + hh * 256;
      bf16x8 pb[1][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f32x4 dtv = *(LDS_AS const f32x4*)(dts + (16 * hf + 8 * e + 4 * hl) * 4);
          const f32x4 dav = *(LDS_AS const f32x4*)(dts + 128 + (16 * hf + 8 * e + 4 * hl) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = raw[hf][e][i >> 1];
            const float cbv = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
            const int kk = k0 + 16 * hf + 8 * e + 4 * hl + i;
            const float decay = __builtin_amdgcn_exp2f((dam[hh] - dav[i]) * kLog2e);
            a[4 * e + i] = kk <= m ? cbv * decay * dtv[i] : 0.f;
          }
        }
        pb[0][hf] = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                           (__bf16)a[4], (__bf16)a[5], (__bf16)a[6], (__bf16)a[7]};
      }
      pv_block<kCsP, kCsBK, 1>(slot + hh * kCsX, off, pb, o[hh]);
    }
  }
  wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  // Output rows through LDS, so that each store instruction writes four whole
  // 256-byte rows: the accumulators hold, per lane, 4-channel groups of one
  // row. All waves have finished with the ring before it is reused. Row r of
  // a wave's 32 x 64 fp32 image keeps its 16-byte chunk c at c ^ (r & 15),
  // so neither the row-wise writes nor the row-major reads conflict.
  block_barrier();
  char* stage = smem + wave * (32 * kCsP * 4);
  const int r = lane & 31, cl = lane & 15;
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    // the image is rewritten per head and read back by other lanes of the
    // same wave: its LDS accesses complete in order; the fences keep the
    // compiler from moving reads above the writes they need or writes above
    // the reads of the previous head
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int t = 0; t < kCsP / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = (t * 32 + g * 8 + hl * 4) / 4;  // 16-byte chunk of the row
        *(LDS_AS f32x4*)(stage + r * (kCsP * 4) + ((ch ^ (r & 15)) << 4)) =
            f32x4{o[hh][0][t][4 * g], o[hh][0][t][4 * g + 1], o[hh][0][t][4 * g + 2], o[hh][0][t][4 * g + 3]};
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 4 * i + (lane >> 4);
      v[i] = *(LDS_AS const f32x4*)(stage + rr * (kCsP * 4) + ((cl ^ (rr & 15)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mm = mw + 4 * i + (lane >> 4);
      // streaming stores: the output is written once and never read back
      // here (2 % faster than plain stores)
      if (mm < Lc)
        __builtin_nontemporal_store(v[i], (f32x4*)(OUT + (((size_t)b * S + c0 + mm) * H + h + hh) * kCsP + 4 * cl));
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
  if (__builtin_mul_overflow((long long)B * S, (long long)H, &rows) ||
      __builtin_mul_overflow(rows, (long long)P, &elems) ||
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
  // two heads per workgroup when the head count is even
  if (H % 2 == 0)
    hipLaunchKernelGGL((chunk_scan_fwd<4, 2>), dim3((unsigned)(groups / 2 * parts)), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t*)x, (const uint16_t*)cb, dt, dA_cumsum, out, S, H, L, nc);
  else
    hipLaunchKernelGGL((chunk_scan_fwd<4, 1>), dim3((unsigned)(groups * parts)), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t*)x, (const uint16_t*)cb, dt, dA_cumsum, out, S, H, L, nc);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
