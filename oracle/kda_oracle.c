/* Plain CPU reference for Kimi Delta Attention (KDA): the gated delta-rule recurrence
 * evaluated token by token, one (sequence, head) chain at a time.
 *
 * TEST INFRASTRUCTURE. This file, and everything under oracle/, is the oracle the
 * HIP path is checked against. Only the tests, the smoke check and the bench's
 * cpu_baseline leg load it; the library never does. It shares no code, header or
 * constant with the HIP path.
 *
 * Two instantiations of the same body:
 *   kda_oracle_f64 - double accumulation; the parity reference.
 *   kda_oracle_f32 - float accumulation; timed as the CPU baseline and used to check
 *                    that the problem is well conditioned.
 * Inputs are passed as float (the exact values of the bf16 or fp32 data the GPU sees),
 * so input rounding is never an error source.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC kda_oracle.c -o libkda_oracle.so -lm
 * (no -ffast-math: the order of every sum is the one written).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

#define REAL double
#define EXP exp
#define FN(x) x##_f64
#include "kda_oracle_body.inc"
#undef REAL
#undef EXP
#undef FN

#define REAL float
#define EXP expf
#define FN(x) x##_f32
#include "kda_oracle_body.inc"
#undef REAL
#undef EXP
#undef FN

int kda_oracle_abi(void) { return 1; }
