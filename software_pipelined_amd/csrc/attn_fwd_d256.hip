// Attention-forward variants for head dimension 256 (see attn_fwd_variants.h).
#define ATTN_FWD_TABLE_TU
#include "attn_fwd_variants.h"

namespace {

// Name fields as in attn_fwd_d64.hip. Default (measured on MI355X): 4-wave
// workgroups (O alone takes 128 registers per lane) with the in-wave
// pipelined schedule and 64-key blocks.
const Variant kTable[] = {
    VARIANT("d256_bm128_bn64_w4_q1_st2_occ1_simple", 256, 4, 64, 1, kSimple, 2, 1, false),
    VARIANT("d256_bm128_bn64_w4_q1_st2_occ1_pipe", 256, 4, 64, 1, kPipelined, 2, 1, true),
    VARIANT("d256_bm128_bn32_w4_q1_st2_occ1_simple", 256, 4, 32, 1, kSimple, 2, 1, false),
    VARIANT("d256_bm128_bn32_w4_q1_st2_occ1_pipe", 256, 4, 32, 1, kPipelined, 2, 1, false),
};
}  // namespace

namespace attn_fwd_impl {

const Variant* variants_d256(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

}  // namespace attn_fwd_impl
