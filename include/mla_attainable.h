/*
 * libmla_attainable -- a measurement aid that ships beside libmla, not part of the decode path.
 *
 * The published matrix-instruction peaks of the MI355X assume the 2.4 GHz peak clock.  Under
 * sustained matrix work the chip holds a lower clock, so a kernel bound by matrix instructions
 * is better read against what the chip sustains.  This library gives that figure: a loop of
 * matrix instructions with no memory traffic, on every compute unit, timed by the caller.
 * Together with a device-to-device copy it gives the attainable rates that a decode kernel's
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

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_ATTAINABLE_H */
