/*
 * fa_rates.h -- instruction-rate loops of the MI355X (gfx950) the attention
 * kernels run on.  Measurement support, not part of the attention path:
 * libfa_rates.so is built beside libfa_mi355x.so and only the benchmark's
 * report calls it, to state the ceilings each forward is measured against.
 *
 * The forward spends, per score element, one FMA (scale and subtract the
 * running maximum), one exponential, one add (row sum), half a max3 (row
 * maximum) and half a bf16 pack on the vector ALU, beside 4 d FLOPs of MFMA
 * work ("flash-attn-triton" docs, Fig. 3: the per-tile update).  At small d
 * that vector work, not the matrix core, bounds the kernel; these loops
 * measure both rates instead of assuming them.
 */
#ifndef FA_RATES_H
#define FA_RATES_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_rates_valu -- seven loops on every compute unit (one workgroup of 8
 * waves per CU, 2 waves per SIMD), each timed with HIP events on `stream`
 * (NULL = the default stream; the call synchronises with it), best of three:
 *   out[0]  dense bf16 MFMA rate, TFLOP/s (v_mfma_f32_32x32x16_bf16, four
 *           independent accumulators per wave)
 *   out[1]  v_exp_f32 rate, 1e12 lane-results per second
 *   out[2]  v_fma_f32 rate, 1e12 lane-results per second
 *   out[3]  the forward's per-score vector sequence above, 1e12 scores/s
 *   out[4]  compute units used
 *   out[5..7]  milliseconds of an interleaved loop -- per step one MFMA and
 *           the per-score sequence of two scores -- with only its MFMAs,
 *           only its vector work, and both: how much of the smaller half
 *           hides under the larger one when the two are independent
 * n is the number of doubles out can hold (at least 8).  The loops touch no
 * memory but one float per lane written to a buffer the call allocates and
 * frees.  Returns 0, -1 for a bad argument, -4 for a HIP error.
 */
int fa_rates_valu(double* out, int n, void* stream);

/*
 * fa_rates_lds -- LDS delivery rate, alone and as MFMA operands.  Each
 * attention kernel feeds every 32x32x16 MFMA one 1 KiB operand read from
 * LDS by its wave; these loops run that pattern on every compute unit (one
 * workgroup of 8 waves per CU, 2 waves per SIMD, a 32 KiB LDS buffer, reads
 * of 16 contiguous bytes per lane, free of bank conflicts), timed like
 * fa_rates_valu:
 *   out[0]  ds_read_b128 alone, TB/s over the whole chip (8 reads in
 *           flight per wave)
 *   out[1]  MFMAs whose A operand is such a read, issued 4 MFMAs ahead,
 *           TFLOP/s
 *   out[2]  the same with the B operand read from LDS too (2 KiB per MFMA)
 *   out[3]  the same number of MFMAs with both operands in registers
 *   out[4]  compute units used
 *   out[5]  milliseconds of the read-only loop
 * n is the number of doubles out can hold (at least 6).  Returns 0, -1 for
 * a bad argument, -4 for a HIP error.
 */
int fa_rates_lds(double* out, int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_RATES_H */
