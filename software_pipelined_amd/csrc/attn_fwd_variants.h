// attn_fwd_variants.h -- the compiled variants of the attention forward:
// each is one kernel schedule at one tiling (head dim, query rows per
// workgroup, keys per block, waves, query tiles per wave, LDS ring slots,
// workgroups per CU). The variant tables live in one translation unit per
// head dimension (attn_fwd_d64.hip, attn_fwd_d128.hip, attn_fwd_d256.hip) so
// that they compile in parallel; attn_fwd.hip holds the C entry points.
#ifndef ATTN_FWD_VARIANTS_H
#define ATTN_FWD_VARIANTS_H

#include <hip/hip_runtime.h>

namespace attn_fwd_impl {

typedef hipError_t (*launch_fn)(const void*, const void*, const void*, float*, float*, int, int, int, int,
                                float, hipStream_t);

struct Variant {
  const char* name;
  int d, bm, bn, waves, lds;
  bool is_default;  // the variant attn_fwd runs for this head dimension (both masks)
  launch_fn fn;
};

// One table per head dimension, defined in attn_fwd_d<d>.hip (host code):
// returns the table and stores its length in *n.
const Variant* variants_d64(int* n);
const Variant* variants_d128(int* n);
const Variant* variants_d256(int* n);

}  // namespace attn_fwd_impl

#ifdef ATTN_FWD_TABLE_TU
// Only the table translation units see the kernels and the launch template.
#include "attn_fwd_kernels.h"

namespace {

using attn_fwd_impl::Variant;

enum Schedule { kSimple = 0, kPipelined = 1, kPingPong = 2, kPingPongFused = 3, kPingPongPre = 4, kPingPong1 = 5 };

// Launch one variant; the scale reaches the kernel as scale_args gives it.
template <int D, int NW, int BN, int QT, int SCHED, int ST, int OCC = 1>
hipError_t launch(const void* q, const void* k, const void* v, float* out, float* lse, int B,
                  int H, int N, int causal, float scale, hipStream_t stream) {
  using T = Tile<D, NW, BN, QT, ST>;
  const int n_qt = (N + T::BM - 1) / T::BM;
  const long long G = fwd_grid((long long)B * H, n_qt, causal);
  const ScaleArgs sa = scale_args(scale);
  const float c = sa.c_log2;
  const int neg = sa.q_mode;
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  clear_last_hip_error();
  const dim3 grid((unsigned)G), block(NW * 64);
  if constexpr (SCHED == kPingPong || SCHED == kPingPong1) {
    constexpr int SYNC = SCHED == kPingPong ? 2 : 1;
    if (causal)
      hipLaunchKernelGGL((attn_fwd_pingpong<D, NW, BN, QT, true, OCC, SYNC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
    else
      hipLaunchKernelGGL((attn_fwd_pingpong<D, NW, BN, QT, false, OCC, SYNC>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
  } else if constexpr (SCHED == kPingPongFused || SCHED == kPingPongPre) {
    constexpr int PRE = SCHED == kPingPongPre;
    if (causal)
      hipLaunchKernelGGL((attn_fwd_pingpong_fused<D, NW, BN, QT, true, OCC, PRE>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
    else
      hipLaunchKernelGGL((attn_fwd_pingpong_fused<D, NW, BN, QT, false, OCC, PRE>), grid, block, 0, stream, qq, kk, vv, out, lse, N, n_qt, c, neg);
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

#define VARIANT(NAME, D, NW, BN, QT, SCHED, ST, OCC, DFLT)                             \
  Variant {                                                                            \
    NAME, D, 32 * QT * NW, BN, NW, Tile<D, NW, BN, QT, ST>::LDS_BYTES, DFLT,           \
        &launch<D, NW, BN, QT, SCHED, ST, OCC>                                         \
  }

}  // namespace
#endif  // ATTN_FWD_TABLE_TU

#endif  // ATTN_FWD_VARIANTS_H
