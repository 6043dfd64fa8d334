// Attention-forward variants for head dimension 128 (see attn_fwd_variants.h).
#define ATTN_FWD_TABLE_TU
#include "attn_fwd_variants.h"

namespace {

// Name fields as in attn_fwd_d64.hip. Default (measured on MI355X): the
// 8-wave ping-pong with 128-key blocks (one barrier pair per 128 keys).
const Variant kTable[] = {
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_simple", 128, 8, 64, 1, kSimple, 2, 1, false),
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_simple", 128, 8, 128, 1, kSimple, 2, 1, false),
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_pingpong", 128, 8, 128, 1, kPingPong, 2, 1, true),
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_ppfused", 128, 8, 128, 1, kPingPongFused, 2, 1, false),
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_ppfusedpre", 128, 8, 128, 1, kPingPongPre, 2, 1, false),
    VARIANT("d128_bm256_bn128_w8_q1_st2_occ1_pingpong1", 128, 8, 128, 1, kPingPong1, 2, 1, false),
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_pingpong", 128, 8, 64, 1, kPingPong, 2, 1, false),
    VARIANT("d128_bm256_bn64_w8_q1_st2_occ1_pingpong1", 128, 8, 64, 1, kPingPong1, 2, 1, false),
    VARIANT("d128_bm256_bn64_w4_q2_st2_occ1_simple", 128, 4, 64, 2, kSimple, 2, 1, false),
    VARIANT("d128_bm128_bn64_w4_q1_st2_occ2_pipe", 128, 4, 64, 1, kPipelined, 2, 2, false),
};
}  // namespace

namespace attn_fwd_impl {

const Variant* variants_d128(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

}  // namespace attn_fwd_impl
