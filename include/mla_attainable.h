/*
 * libmla_attainable -- a measurement aid that ships beside libmla, not part of the decode path.
 *
 * The published matrix-instruction peaks of the MI355X assume the 2.4 GHz peak clock.  Under
 * sustained matrix work the chip holds a lower clock, so a kernel bound by matrix instructions
 * is better read against what the chip sustains.  This library gives that figure: a loop of
 * matrix instructions with no memory traffic, on every compute unit, timed by the caller.
 * Two read-only streams of a device buffer give the HBM read bandwidth the chip sustains, one
 * with plain vector loads and one with the buffer->LDS loads and LDS ring of the decode split.
 * Together with a device-to-device copy they give the attainable rates that a decode kernel's
 * roofline fraction can be read against.
 */
#ifndef LIBMLA_ATTAINABLE_H
#define LIBMLA_ATTAINABLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix instructions the loop can issue, with the floating-point operations each performs. */
typedef enum {
  MLA_LOOP_BF16 = 0, /* v_mfma_f32_32x32x16_bf16: 32 x 32 x 16 x 2 = 32,768 FLOP */
  MLA_LOOP_FP8 = 1   /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 operands, unit block scales:
                        32 x 32 x 64 x 2 = 131,072 FLOP */
} mla_loop_kind_t;

/*
 * mla_attainable_mfma_loop -- launch `workgroups` workgroups of 256 threads (four waves, one
 * per SIMD when a compute unit holds one workgroup).  Every wave issues iters x 4 instructions
 * of `kind` in four independent accumulation chains, so no instruction waits on the one
 * before it; operands are fixed pseudo-random values held in registers.  Each workgroup
 * reserves `lds_bytes` of LDS (0 .. 163840): 163840 keeps one workgroup per compute unit (the
 * decode split's occupancy), 81920 allows two.  Total FLOP = workgroups * 4 * iters * 4 * (FLOP
 * per instruction above).
 *   out  [workgroups * 256] fp32, device, 16-byte aligned: each thread's accumulator sum,
 *        written so that the loop is not removed (its value carries no meaning).
 * Asynchronous on `stream` (a hipStream_t; NULL is the default stream).  Returns 0; -1 for an
 * argument out of range (nothing launched; checked before any HIP call); otherwise the HIP
 * error code of the failed call.
 */
int32_t mla_attainable_mfma_loop(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes, float* out,
                                 void* stream);

/* Ways a read stream brings the buffer in. */
typedef enum {
  MLA_READ_VGPR = 0, /* 16-byte vector loads into registers (non-temporal), nine per chunk and
                        lane, issued before they are summed; any number of workgroups per CU */
  MLA_READ_LDS = 1   /* 16-byte buffer->LDS loads (1 KiB per wave instruction) into a ring of
                        four 36,864-byte LDS stages, three chunks in flight, one barrier per
                        chunk: the decode split's loads without its arithmetic; all of a
                        compute unit's LDS (147,456 B) per workgroup, so one per CU */
} mla_read_kind_t;

/*
 * mla_attainable_read -- read `bytes` of `buf` once.  The buffer is cut into chunks of 36,864 B
 * (a half page of the bf16 decode split); workgroup w (of `workgroups`, 256 threads each) reads
 * the contiguous chunks w*n .. w*n+n-1, n = bytes / (workgroups * 36864).  Every 32-bit word
 * is read by exactly one thread, which adds it into a wrapping 32-bit sum.
 *   buf  device, 256-byte aligned, `bytes` long; bytes must be a multiple of
 *        workgroups * 36864, and one workgroup's slice below 2^31 bytes.
 *   out  [workgroups * 256] uint32, device, 16-byte aligned: each thread's sum.  The sum of
 *        all of them equals the sum of the buffer's 32-bit words mod 2^32.
 * Bytes read / time is the read bandwidth.  Asynchronous on `stream` (a hipStream_t; NULL is
 * the default stream).  Returns 0; -1 for an argument out of range (nothing launched; checked
 * before any HIP call); otherwise the HIP error code of the failed call.
 */
int32_t mla_attainable_read(int32_t kind, const void* buf, int64_t bytes, int32_t workgroups, uint32_t* out,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_ATTAINABLE_H */
