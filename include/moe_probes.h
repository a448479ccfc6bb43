/*
 * moe_probes.h -- measurement probes exported by libmoe.so next to the layer's
 * entry points (include/moe.h).  They are not part of the layer: they measure
 * the practical ceilings that the layer's kernels are compared with (an HBM
 * streaming read, an MFMA-only loop and the decode kernel's all-to-all
 * hand-offs on their own), on the caller's stream, with the
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

/* One all-to-all hand-off of the persistent decode kernel, repeated `rounds`
 * times with no other work: one 512-thread workgroup per CU
 * (moe_probe_exchange_blocks() of them, all resident), tagged 8-byte words,
 * relaxed agent-scope stores and loads, every thread polling its own words,
 * one barrier per round.  pattern 0: x (each workgroup publishes its share
 * of 2,048 words to 8 per-XCD copies, every workgroup reads the 2,048 words
 * of its XCD's copy); 1: logits (512 words, likewise); 2: partial sums (each
 * workgroup writes 2,048 words and reads its 2,048 / G rows of all G).
 * ws: moe_probe_exchange_ws_bytes() bytes (cleared by the probe); ticks:
 * int64 [moe_probe_exchange_blocks()] out, the 100 MHz wall-clock ticks each
 * workgroup spent; err: int32 [1] out, the number of workgroups whose wait
 * ran past its bound (0 when every round completed).  Needs a CU count that
 * divides 512; MOE_EUNSUPPORTED otherwise or when the workgroups cannot all be
 * resident. */
int moe_probe_exchange(int pattern, int rounds, void* ws, size_t ws_bytes, long long* ticks, int* err, void* stream);
int moe_probe_exchange_blocks(void);
size_t moe_probe_exchange_ws_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBES_H */
