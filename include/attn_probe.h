/*
 * attn_probe.h -- a measurement entry point of libattn.so (not an operator).
 *
 * attn_probe_mfma runs a stream of bf16 matrix-core instructions on
 * `blocks` workgroups of 4 waves: every wave issues iters x 16 of them over
 * 4 independent accumulators, with
 *     mode 0 : v_mfma_f32_32x32x16_bf16 (32,768 flops), both operands in
 *              registers,
 *     mode 1 : the same, one operand read from LDS for every instruction
 *              (16 bytes per lane, 1 KiB per wave: the attention kernels'
 *              ratio of LDS bytes to matrix work),
 *     mode 2 : v_mfma_f32_16x16x32_bf16 (16,384 flops), operands in
 *              registers,
 *     mode 3 : mode 2 with one 1 KiB LDS read per instruction (twice the
 *              LDS bytes per flop of mode 1).
 * Timing it (and reading the shader clock from counters) gives the matrix
 * rate and clock the card sustains for each kind of stream, and with mode 3
 * the LDS read rate a 16x16x32 stream can draw. Work per call =
 * blocks * 4 * iters * 16 * F flops, F = 32768 (modes 0, 1) or 16384
 * (modes 2, 3).
 *
 *   out    : device, float32, blocks * 256 values (a sum per thread, written
 *            so that the work is observable; their values carry no meaning)
 *   blocks : 1 .. 2^20; iters >= 1; mode 0 .. 3 (else ATTN_ERR_BAD_SHAPE)
 *   stream : hipStream_t (NULL = default stream); one kernel is enqueued
 *
 * Returns ATTN_OK, ATTN_ERR_BAD_SHAPE, ATTN_ERR_NULL_PTR or ATTN_ERR_HIP
 * (codes of attn.h). Asynchronous; allocates nothing.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

int attn_probe_mfma(int mode, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
