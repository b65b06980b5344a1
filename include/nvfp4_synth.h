/*
 * nvfp4_synth.h — seeded synthetic expert weights generated on the device.
 * Input generation for tests and benchmarks only; it is not part of the MoE
 * layer and shares nothing with it.
 *
 * Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11), key (seed, tag), counter
 * (i / 4, expert, 0, 0) for element i of an expert (output word i % 4).  The
 * word's four 16-bit fields are summed and centred (Irwin-Hall of order 4,
 * range +-131070) and multiplied in binary32 by
 * nvfp4_synth_scale(sigma) = (float)(sigma / sqrt(4 (2^32 - 1) / 12)),
 * giving values of standard deviation sigma.
 */
#ifndef NVFP4_SYNTH_H
#define NVFP4_SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fill out_dev f32 [experts, n_per_expert] (16-byte aligned) with experts
 * expert0 .. expert0+experts-1.  experts <= 65535.  Returns 0 on success,
 * 1 for a bad argument, 6 for a HIP launch error.  Asynchronous on stream. */
int nvfp4_synth_weights(uint64_t seed, uint64_t tag, int64_t expert0, int64_t experts,
                        int64_t n_per_expert, double sigma, float* out_dev, void* stream);

float nvfp4_synth_scale(double sigma);

const char* nvfp4_synth_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_SYNTH_H */
