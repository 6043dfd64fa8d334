// Attention-forward variants for head dimension 64 (see attn_fwd_variants.h).
#define ATTN_FWD_TABLE_TU
#include "attn_fwd_variants.h"

namespace {

// Name fields: head dim, query rows per workgroup, keys per block, waves,
// query tiles per wave, LDS ring slots, workgroups per CU (occ), schedule.
// Default (measured on MI355X): 4-wave workgroups with two query tiles per
// wave (every K/V fragment read feeds two MFMAs), two workgroups per CU.
const Variant kTable[] = {
    VARIANT("d64_bm256_bn64_w8_q1_st2_occ1_simple", 64, 8, 64, 1, kSimple, 2, 1, false),
    VARIANT("d64_bm256_bn64_w4_q2_st2_occ2_simple", 64, 4, 64, 2, kSimple, 2, 2, true),
    VARIANT("d64_bm128_bn64_w4_q1_st2_occ3_pipe", 64, 4, 64, 1, kPipelined, 2, 3, false),
    VARIANT("d64_bm128_bn128_w4_q1_st2_occ2_simple", 64, 4, 128, 1, kSimple, 2, 2, false),
    VARIANT("d64_bm256_bn128_w4_q2_st2_occ1_simple", 64, 4, 128, 2, kSimple, 2, 1, false),
    VARIANT("d64_bm256_bn128_w8_q1_st2_occ1_pingpong1", 64, 8, 128, 1, kPingPong1, 2, 1, false),
};
}  // namespace

namespace attn_fwd_impl {

const Variant* variants_d64(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

}  // namespace attn_fwd_impl
