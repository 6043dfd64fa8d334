// Fused attention forward for MI355X (gfx950, CDNA4), behind the C ABI in
// include/attn.h: the C entry points. The kernels are in attn_fwd_kernels.h,
// the variant tables in attn_fwd_d64.hip, attn_fwd_d128.hip, attn_fwd_d256.hip.
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
// wgmma warp groups are prior art):
//   * a workgroup has NW wavefronts; each wave owns QT tiles of 32 query
//     rows end to end (BM = 32*QT*NW rows per workgroup);
//   * S is formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K (from LDS) is the A operand and Q^T (kept in registers for the whole
//     loop) the B operand, so each lane's accumulator column is one query and
//     row max / row sum reduce within the lane plus one lane^32 swap
//     (v_permlane32_swap); with QT = 2 every K fragment read from LDS feeds
//     two MFMAs;
//   * O^T += V^T P^T with the same instruction: P^T goes straight from the
//     S accumulators into the B operand (cvt to bf16, no LDS round trip),
//     V^T is read with the gfx950 transposing LDS read ds_read_b64_tr_b16;
//   * K/V blocks stream through an LDS ring filled with
//     buffer_load_dwordx4 ... lds (HBM -> LDS without VGPRs); the destination
//     layout is XOR-swizzled per row by choosing which global chunk each lane
//     fetches, so MFMA fragment reads are bank-conflict free;
//   * exp2 runs on v_exp_f32 with scale*log2(e) folded into one FMA;
//   * the O *= alpha rescale is skipped by a whole wave when none of its
//     rows raised its running max in the block (alpha == 1 exactly). The max
//     itself is tracked exactly, never lazily: a stale max makes the
//     dominant key's weight 2^delta instead of exactly 1, and its bf16
//     rounding then costs up to 2^-9 |v| on near-one-hot rows;
//   * workgroup ids are remapped so that consecutive query tiles of one head
//     run on one XCD (shared L2 for that head's K/V); causal grids start with
//     the heaviest tiles.
// Three schedules share the per-block step helpers (same arithmetic, bit for
// bit): "simple" (steps in program order), "pingpong" (two wave groups take
// turns on the matrix core) and "pipe" (each wave overlaps the softmax of
// block j with the QK^T MFMAs of block j+1).

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include "attn.h"
#include "attn_fwd_variants.h"

namespace {

using attn_fwd_impl::Variant;

// Variant ids run through the d = 64, 128 and 256 tables in that order.
struct Table {
  const Variant* v;
  int n;
};
Table table(int i) {
  Table t;
  t.v = i == 0 ? attn_fwd_impl::variants_d64(&t.n)
               : i == 1 ? attn_fwd_impl::variants_d128(&t.n) : attn_fwd_impl::variants_d256(&t.n);
  return t;
}
int num_variants() { return table(0).n + table(1).n + table(2).n; }
const Variant* variant(int id) {
  if (id < 0) return nullptr;
  for (int i = 0; i < 3; ++i) {
    const Table t = table(i);
    if (id < t.n) return t.v + id;
    id -= t.n;
  }
  return nullptr;
}

// The measured default per head dimension (the same for both masks).
int default_variant(int d, int causal) {
  (void)causal;
  for (int id = 0, n = num_variants(); id < n; ++id) {
    const Variant* v = variant(id);
    if (v->d == d && v->is_default) return id;
  }
  return -1;
}

int validate(const void* q, const void* k, const void* v, const float* out, const float* lse,
             int B, int H, int N, int d, float scale, int bm) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  uint32_t sbits;
  memcpy(&sbits, &scale, sizeof sbits);  // bit test: immune to fast-math folding
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_BAD_SCALE;  // NaN or +-Inf
  long long bh = 0, rows = 0, elems = 0, grid = 0;
  if (__builtin_mul_overflow((long long)B, (long long)H, &bh) ||
      __builtin_mul_overflow(bh, (long long)N, &rows) ||
      __builtin_mul_overflow(rows, (long long)d, &elems) ||
      __builtin_mul_overflow(bh, (long long)((N + bm - 1) / bm), &grid))
    return ATTN_ERR_BAD_SHAPE;
  if (rows == 0) return ATTN_OK;
  // element offsets are 64-bit in the kernel; the grid is one dimension
  // (a dispatch counts work-items in 32 bits: workgroups x 512 threads < 2^32)
  if (elems > (1LL << 50) || grid > 0xFFFFFFFFLL / 512) return ATTN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_PTR;
  const uintptr_t m = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if ((m & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

int run_variant(int id, const void* q, const void* k, const void* v, float* out, float* lse, int B,
                int H, int N, int d, int causal, float scale, void* stream) {
  const Variant* var = variant(id);
  if (!var) return ATTN_ERR_BAD_SHAPE;
  int st = validate(q, k, v, out, lse, B, H, N, d, scale, var->bm);
  if (st != ATTN_OK) return st;
  if (var->d != d) return ATTN_ERR_BAD_SHAPE;
  if (B == 0 || H == 0 || N == 0) return ATTN_OK;
  hipError_t e = var->fn(q, k, v, out, lse, B, H, N, causal, scale, (hipStream_t)stream);
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
    case ATTN_ERR_BAD_SHAPE: return "bad shape (negative size, size overflow, or a variant id that is out of range or serves another head dimension)";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension";
    case ATTN_ERR_BAD_SCALE: return "scale must be finite";
    case ATTN_ERR_MISALIGNED: return "pointer misaligned (16 bytes; 4 for lse and the backward's per-row statistics)";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than the entry point's workspace-size function reports";
    case ATTN_ERR_TOO_LARGE: return "shape needs more scratch than the no-allocation entry's fixed buffer holds";
    default: return "unknown status";
  }
}

int attn_num_variants(void) { return num_variants(); }

const char* attn_variant_name(int id) {
  const Variant* v = variant(id);
  return v ? v->name : nullptr;
}

int attn_variant_info(int id, int* head_dim, int* block_m, int* block_n, int* waves,
                      int* lds_bytes) {
  const Variant* v = variant(id);
  if (!v) return ATTN_ERR_BAD_SHAPE;
  if (head_dim) *head_dim = v->d;
  if (block_m) *block_m = v->bm;
  if (block_n) *block_n = v->bn;
  if (waves) *waves = v->waves;
  if (lds_bytes) *lds_bytes = v->lds;
  return ATTN_OK;
}

int attn_default_variant(int d, int causal) { return default_variant(d, causal); }

int attn_fwd_variant(int id, const void* q, const void* k, const void* v, float* out, float* lse,
                     int B, int H, int N, int d, int causal, float scale, void* stream) {
  return run_variant(id, q, k, v, out, lse, B, H, N, d, causal, scale, stream);
}

}  // extern "C"
