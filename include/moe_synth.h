/*
 * moe_synth.h - seeded synthetic expert weights, generated on the GPU.
 *
 * Benchmark and test input generator, not part of the MoE method: it fills
 * expert blobs (byte layout in moe.h) with the same values as the host
 * generator of the test-suite, bit for bit, so that the 43.5 GB of an
 * 80B-shaped expert table can be produced in HBM in seconds while any single
 * expert can still be regenerated on the host.
 *
 * Definition (Philox4x32-10 of Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC'11):
 *   key     = (seed & 0xffffffff, layer)
 *   counter = (block, expert_id, tensor, 0); tensor 0/1/2 = gate/up/down
 *             nibbles, 3/4/5 = gate/up/down scales
 *   nibbles: value j = r*cols + c of a [rows][cols] matrix is bits
 *            [4*(j%8), 4*(j%8)+4) of output word (j%32)/8 of block j/32
 *   bytes:   (int8 experts) value j is bits [8*(j%4), 8*(j%4)+8) of output
 *            word (j%16)/4 of block j/16
 *   scales:  value j = r*(cols/G) + g uses output word j%4 of block j/4;
 *            u = (word >> 8) * 2^-24, s = fp16_rne((u * scale_span) + scale_lo)
 *            with both fp32 operations rounded separately (no fused
 *            multiply-add), and bias b = -8 * s for int4, -128 * s for int8
 *            (exact either way).
 */
#ifndef MOE_AMD_MOE_SYNTH_H
#define MOE_AMD_MOE_SYNTH_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Fill n_experts blobs of weight_bits 4 or 8: blob k (expert id
 * expert_first + k) is written at dst + k*stride (device, 256-byte aligned,
 * stride a multiple of 256 and at least moe_blob_bytes_q(hidden, inter,
 * group_size, weight_bits)).  The shared expert of a layer with E routed
 * experts uses expert id E (and its own inter).  MOE_ESHAPE for unsupported
 * sizes or widths, MOE_EINVAL for a bad destination. */
moe_status moe_synth_fill_experts(uint64_t seed, int32_t layer, int32_t expert_first, int32_t n_experts,
                                  int32_t hidden, int32_t inter, int32_t group_size, int32_t weight_bits,
                                  float scale_lo, float scale_span, uint8_t* dst, uint64_t stride,
                                  moe_stream stream);

/* The first four output words of Philox4x32-10 for each of n counters
 * (device arrays ctr [n][4], key [n][2], out [n][4]); used to check the
 * device generator against published known-answer vectors. */
moe_status moe_synth_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_SYNTH_H */
