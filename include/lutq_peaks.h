/*
 * lutq peaks -- microbenchmarks of the GPU that the lutq kernels are
 * measured against (part of liblutq.so). They give the measured floors
 * beside the published ones:
 *   - the cost of one launch with no work, in back-to-back launches;
 *   - a streaming read of a buffer, in the fastest shape tried on MI355X,
 *     with or without a small store at the end (as a matmul that writes y);
 *   - the fp16 MFMA issue rate of the two gfx950 shapes the kernels can use;
 *   - the rate of random 32-bit LDS reads, the access of the on-chip lookup
 *     table (FLUTE abstract: shared-memory bandwidth is what the
 *     vectorized, duplicated table is designed around).
 *
 * Each call validates its arguments, then enqueues one launch on `stream`
 * (a hipStream_t as void*, NULL = default stream) and returns LUTQ_OK, or a
 * negative lutq status (include/lutq.h) with nothing enqueued. Timing is
 * the caller's: replay many launches (a HIP graph) between events recorded
 * on the same stream and divide by the count. Sinks are caller-owned
 * device buffers that receive results no one reads.
 */
#ifndef LUTQ_PEAKS_H
#define LUTQ_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One launch of an empty kernel (1 workgroup of 64 threads). */
int lutq_peak_empty(void* stream);

/* Bytes the `sink` of lutq_peak_stream must hold (16-byte aligned). */
size_t lutq_peak_stream_sink_bytes(void);

/* Reads `bytes` bytes at `buf` (device, 16-byte aligned, bytes a multiple
 * of 16 and > 0) once, 16 bytes per lane and sweep over 2048 workgroups of
 * 256 threads, with nontemporal loads. store != 0: every wave then writes
 * 16 bytes to `sink`. Bytes moved per launch: `bytes` read (+ 128 KiB
 * written with store). Errors: LUTQ_EINVAL, LUTQ_EALIGN, LUTQ_EHIP. */
int lutq_peak_stream(const void* buf, size_t bytes, int store, uint32_t* sink, void* stream);

/* fp16 MFMA issue rate: one workgroup per compute unit with
 * 4 * waves_per_simd waves (1..4 per SIMD); each wave runs `iters` rounds
 * of independent MFMAs worth 131072 floating-point operations per round:
 * eight v_mfma_f32_16x16x32_f16 (kind LUTQ_PEAK_MFMA_16X16X32) or four
 * v_mfma_f32_32x32x16_f16 (LUTQ_PEAK_MFMA_32X32X16). FLOPs per launch =
 * CUs * 4 * waves_per_simd * iters * 131072. `sink`: device, fp32, at least
 * CUs * 16 entries. Errors: LUTQ_EINVAL, LUTQ_EHIP. */
enum { LUTQ_PEAK_MFMA_16X16X32 = 0, LUTQ_PEAK_MFMA_32X32X16 = 1 };
int lutq_peak_mfma(int kind, int waves_per_simd, int iters, float* sink, void* stream);

/* 32-bit LDS reads in the access pattern of the lutq pair table (256
 * entries of 64 copies, 64 KiB; lane L reads copy L of its entry, so an
 * instruction's 64 lanes hit 64 distinct banks): one workgroup of
 * waves_per_cu waves (1..16) per compute unit; each lane holds 16 random
 * entries and reads them all every round, one ds_read_b32 each (16 in
 * flight), `iters` rounds. Wave-wide ds_read_b32 instructions per launch =
 * CUs * waves_per_cu * 16 * iters.
 * `sink`: device, one uint32. Errors: LUTQ_EINVAL, LUTQ_EHIP. */
int lutq_peak_lds(int waves_per_cu, int iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LUTQ_PEAKS_H */
