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

/*
 * fa_rates_atomic -- the cost of accumulating dQ with atomics inside the
 * dK/dV kernel, the alternative to a separate dQ kernel that recomputes S
 * and dP (the pages leave open how dQ is accumulated: "flash-attn-triton"
 * docs, "Where things live").  Runs the accumulation alone, in the pattern
 * that form would issue for BH heads of N rows at d = 128 under the causal
 * mask: one workgroup per (128-key block, head) adds a 32 x 128 float32 tile
 * for every 32-row query tile its block sees, with hardware float32 atomic
 * adds; then checks every sum (each row counted once per block that sees
 * it).  Best of three, timed with HIP events on `stream` (synchronised):
 *   out[0]  bytes of float32 added
 *   out[1]  ms, head index fastest in the grid (a head's blocks on one XCD)
 *   out[2]  ms, key block fastest (a head's blocks spread over every XCD)
 *   out[3]  ms of the same traffic as plain read-add-write (not atomic)
 *   out[4]  TB/s of atomic adds in the first ordering
 *   out[5], out[6]  wrong sums in the two orderings (0 expected)
 *   out[7]  TB/s of the plain reference
 * Needs N a multiple of 128, BH * N * 128 <= 2^30, n >= 8; allocates and
 * frees a BH * N * 128 float buffer and a host copy.  Returns 0, -1 for a
 * bad argument, -4 for a HIP or host allocation error.
 */
int fa_rates_atomic(double* out, int n, int N, int BH, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_RATES_H */
