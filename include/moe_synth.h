/*
 * moe_synth.h -- C-ABI of libmoe_synth.so: the seeded synthetic-input generator on the GPU.
 * Test and benchmark harness, not part of the layer: it fills device buffers with the same
 * values as the host generator (synth/generator.py), bit for bit.
 *
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC 2011) on the counter (i mod 2^32, i div 2^32, c2, c3) under the key (seed, 0x4D6F4531);
 * the eight 16-bit halves of the output are summed (Irwin-Hall), centred (-262140) and
 * multiplied by `scale` in fp32: out[j] = fp32(sum16(philox(start + j)) - 262140) * scale.
 */
#ifndef MOE_SYNTH_H
#define MOE_SYNTH_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* out [n] fp32 device buffer (16-byte aligned not required).  Returns 0 on success, a HIP
 * error code otherwise; n <= 0 enqueues nothing. */
int32_t synth_normal_f32(float *out, int64_t n, uint64_t start, uint32_t seed, uint32_t c2,
                         uint32_t c3, float scale, hipStream_t stream);

/* Raw Philox4x32-10 words for the counters i = start + j (low word, high word, c2, c3):
 * out[4j .. 4j+3] = philox(ctr = (i lo, i hi, c2, c3), key = (seed, key1)).  For checks. */
int32_t synth_philox_words(uint32_t *out, int64_t n, uint64_t start, uint32_t seed,
                           uint32_t key1, uint32_t c2, uint32_t c3, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
