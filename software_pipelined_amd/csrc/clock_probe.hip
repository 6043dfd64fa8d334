// clock_probe.hip -- a measurement kernel of libattn.so: the matrix-core rate
// and shader clock the card sustains for a stream of bf16 MFMAs (32x32x16 or
// 16x16x32), with the operands in registers or with one 1 KiB LDS read per
// MFMA. Not part of any operator; the C ABI is declared in
// include/attn_probe.h.

#include "attn_common.h"
#include "attn_probe.h"

namespace {

constexpr int kProbeChains = 4;  // independent accumulators: back-to-back MFMA issue
constexpr int kProbeUnroll = 16;
constexpr int kProbeLdsBytes = 64 * 1024;  // 16 KiB per wave: 16 distinct 1 KiB reads per pass

// One workgroup of 4 waves (one per SIMD). Each wave runs iters x 16 MFMAs
// (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_16x16x32_bf16 with SMALL: half
// the work per instruction, same operand size) over kProbeChains
// accumulators; with LDS, every MFMA's A operand is a fresh
// 16-byte-per-lane LDS read (1 KiB per wave; the address moves with the
// iteration, so no read is loop-invariant), issued 8 MFMAs ahead. The
// accumulators are summed and stored so that the work cannot be dropped.
template <bool LDS, bool SMALL>
__global__ __launch_bounds__(256) void mfma_clock_probe(float* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(1024))) char smem[kProbeLdsBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // small finite bf16 values (the products stay finite over any run length)
  for (int i = threadIdx.x; i < kProbeLdsBytes / 16; i += 256) {
    const float v = (float)((i & 7) - 3) * 0.0078125f;
    *(LDS_AS bf16x8*)(smem + 16 * i) =
        bf16x8{(__bf16)v, (__bf16)(-v), (__bf16)v, (__bf16)v, (__bf16)(-v), (__bf16)v, (__bf16)(-v), (__bf16)v};
  }
  __syncthreads();
  const float fa = (float)((lane & 3) - 1) * 0.0078125f, fb = (float)((lane >> 4) - 2) * 0.0078125f;
  const bf16x8 a0 = {(__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb};
  const bf16x8 b0 = {(__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa};
  using acc_t = typename std::conditional<SMALL, f32x4, f32x16>::type;
  acc_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = acc_t{};
  auto mfma = [&](const bf16x8& a, acc_t& c) {
    if constexpr (SMALL)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, c, 0, 0, 0);
    else
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, c, 0, 0, 0);
  };
  // each wave walks its own 16 KiB quarter of the LDS image, 1 KiB per read
  const char* base = smem + wave * (kProbeLdsBytes / 4) + lane * 16;
  for (int it = 0; it < iters; ++it) {
    if constexpr (LDS) {
      bf16x8 fr[kProbeUnroll];
#pragma unroll
      for (int k = 0; k < kProbeUnroll; ++k) fr[k] = *(LDS_AS const bf16x8*)(base + (((k + it) & 15) << 10));
#pragma unroll
      for (int k = 0; k < kProbeUnroll; ++k) mfma(fr[k], acc[k % kProbeChains]);
      sched_mfma_with_reads<kProbeUnroll, 1, 1, 8>();
    } else {
#pragma unroll
      for (int k = 0; k < kProbeUnroll; ++k) mfma(a0, acc[k % kProbeChains]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < (SMALL ? 4 : 16); ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int attn_probe_mfma(int mode, int blocks, int iters, float* out, void* stream) {
  if (mode < 0 || mode > 3 || blocks < 1 || iters < 1 || blocks > (1 << 20)) return ATTN_ERR_BAD_SHAPE;
  if (!out) return ATTN_ERR_NULL_PTR;
  clear_last_hip_error();
  const hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL((mfma_clock_probe<false, false>), dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL((mfma_clock_probe<true, false>), dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL((mfma_clock_probe<false, true>), dim3(blocks), dim3(256), 0, st, out, iters); break;
    default: hipLaunchKernelGGL((mfma_clock_probe<true, true>), dim3(blocks), dim3(256), 0, st, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
