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

/*
 * Matrix-core throughput with one operand from LDS, as in the attention
 * kernel's inner loop: `blocks` workgroups of 512 work-items (8 wavefronts,
 * one workgroup per compute unit), each wavefront running `iters` iterations
 * of 8 v_mfma_f32_32x32x16_bf16 products, each taking a fresh 1 KB fragment
 * read from LDS (16 bytes per lane) and a register operand, in two
 * accumulation chains.  Work = blocks * 8 * iters * 8 * 32768 FLOP.  sink
 * (device, blocks * 512 floats) receives one float per work-item.  Returns 0,
 * 1 for bad arguments, or 8 when the launch fails.
 */
int32_t bwa_probe_mfma_lds_bf16(int32_t iters, int32_t blocks, float* sink, void* stream);

/*
 * The same with a chosen mix of LDS operand reads per pair of products:
 * n_b128 reads of 16 bytes per lane (1 KB each) and n_tr pairs of
 * transposing 8-byte reads (ds_read_b64_tr_b16, 1 KB per pair), combined into
 * the A operand of both products of the pair; each wavefront runs `iters`
 * iterations of 4 pairs.  Work = blocks * 8 * iters * 8 * 32768 FLOP.  The
 * mixes built are (n_b128, n_tr) = (2, 0), (0, 2), (1, 1), (2, 1), (4, 0),
 * (3, 1) and (6, 0).  Returns 0, 1 for bad arguments or a mix not built, or
 * 8 when the launch fails.
 */
int32_t bwa_probe_mfma_lds_mix(int32_t n_b128, int32_t n_tr, int32_t iters, int32_t blocks, float* sink,
                               void* stream);

/*
 * HBM streaming probe: the bandwidth the device sustains for a mix of
 * reads and writes.  src (device, 16-byte aligned) holds `ratio` streams of
 * `chunks` 16-byte chunks each; every chunk is read once with non-temporal
 * loads.  With dst (device, 16-byte aligned, `chunks` 16-byte chunks), chunk j
 * of dst receives the XOR of chunk j of every stream: ratio * 16 bytes read
 * per 16 bytes written (the LSE merge of two fp32 partials into bf16 reads
 * 4 bytes per byte written).  With dst NULL nothing but sink (device, one
 * float per work-item) is written: a read-only pass.  `blocks` workgroups of
 * 256 work-items stride over the chunks.  Returns 0, 1 for bad arguments,
 * or 8 when the launch fails.
 */
int32_t bwa_probe_stream(const void* src, int64_t chunks, int32_t ratio, void* dst, int32_t blocks, float* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BWA_PROBE_H */
