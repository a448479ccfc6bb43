/*
 * moe_probes.h -- measurement probes exported by libmoe.so next to the layer's
 * entry points (include/moe.h).  They are not part of the layer: they measure
 * the practical ceilings that the layer's kernels are compared with (an HBM
 * streaming read and an MFMA-only loop), on the caller's stream, with the
 * conventions of moe.h (device pointers owned by the caller, MOE_OK or a
 * negative code, moe_last_error()).
 */
#ifndef MOE_PROBES_H
#define MOE_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` once with 16-byte loads spread over the whole
 * device and writes one fold of the data per workgroup to sink (so the reads
 * cannot be dropped).  src 16-byte aligned, bytes a multiple of 16;
 * sink: uint32 [moe_probe_stream_read_blocks()]. */
int moe_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
int moe_probe_stream_read_blocks(void);

/* Runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_f16 chains per
 * wave on register operands (no memory traffic) over 256 workgroups of 4
 * waves per compute unit, and writes one sum per workgroup to sink (fp32
 * [moe_probe_mfma_blocks()]).  Floating-point work: 4 * 32768 flop per wave
 * per round; moe_probe_mfma_flops(iters) returns the total. */
int moe_probe_mfma(int iters, float* sink, void* stream);
int moe_probe_mfma_blocks(void);
double moe_probe_mfma_flops(int iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBES_H */
