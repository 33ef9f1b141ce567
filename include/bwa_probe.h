/*
 * bwa_probe.h -- measurement helper shipped beside the attention library
 * (libbwa_probe.so, gfx950).  It is not part of the attention method: it
 * measures what the matrix cores of the device sustain, so that attention
 * throughput can be stated against a measured ceiling as well as against
 * the published peak.
 *
 * All pointers are device pointers; the call is asynchronous on the stream
 * and allocates nothing.
 */
#ifndef BWA_PROBE_H
#define BWA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launch `blocks` workgroups of 256 work-items (4 wavefronts).  Every
 * wavefront runs `iters` iterations of 4 independent
 * v_mfma_f32_32x32x16_bf16 accumulations on register operands (no memory
 * traffic in the loop), then writes one float per work-item to sink
 * (device, blocks * 256 floats) so that the work cannot be removed.
 * Work = blocks * 4 * iters * 4 * 32768 FLOP.
 * clocks (device, 2 x uint64, may be NULL): for the first wavefront, the
 * shader-clock cycles (s_memtime) and the 100 MHz real-time ticks
 * (s_memrealtime) spent in the loop; their ratio gives the shader clock.
 * Returns 0, 1 for bad arguments (iters < 1, blocks < 1, sink NULL), or
 * 8 when the launch fails.
 */
int32_t bwa_probe_mfma_bf16(int32_t iters, int32_t blocks, float* sink, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BWA_PROBE_H */
