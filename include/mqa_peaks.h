/*
 * mqa_peaks.h -- C ABI of libmqa_peaks.so: probes that measure the ceilings
 * the attention kernels of libmqa_attn.so are measured against, on the device
 * they run on.  The attention pages give no hardware figures; the rooflines
 * of this library's kernels are (a) the dense bf16 MFMA rate (prefill, and
 * MLA decode, whose 240 flop per byte sits near the ridge) and (b) HBM read
 * bandwidth (decode streams its KV cache once: "GQA和MLA详解"
 * (lzwjava.github.io) §1, decode phase bound by memory bandwidth).  A
 * published peak assumes the top clock; these probes report what the same
 * instructions reach at the clock the part actually sustains.
 *
 * Conventions: every pointer is a DEVICE pointer owned by the caller
 * (16-byte aligned where it is a data buffer); each call enqueues one
 * kernel on `stream` (a hipStream_t, NULL = default stream) and returns at
 * once; the caller times it (HIP events).  Return value 0 on success, -1
 * for an invalid argument (nothing enqueued), -4 when the HIP runtime
 * reports a launch error or no device.  `sink` receives a checksum per
 * thread and is otherwise meaningless; size it with mqa_peak_sink_floats().
 */
#ifndef MQA_PEAKS_H
#define MQA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MQA_PEAK_MFMA = 0, MQA_PEAK_READ = 1, MQA_PEAK_LDS = 2 };

/* Compute units of the current device (0 if the query fails). */
int mqa_peak_compute_units(void);

/* Floats the `sink` of the given probe kind needs (MQA_PEAK_MFMA with
 * waves_per_simd 1 or 2; MQA_PEAK_READ also covers mqa_peak_hbm_copy's
 * launch shape; MQA_PEAK_LDS for any waves_per_cu). */
size_t mqa_peak_sink_floats(int kind, int waves_per_simd);

/* One workgroup per compute unit, waves_per_simd (1 or 2) waves on each of
 * its 4 SIMDs; each wave issues iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 flop each).  Total flop =
 * CUs x 4 x waves_per_simd x iters x 8 x 32768.  clocks[0] receives the
 * shader-clock cycles (s_memtime) and clocks[1] the 100 MHz real-time ticks
 * (s_memrealtime) that one wave spent in its loop: their ratio x 100 MHz is
 * the clock the loop ran at.  clocks: 2 x uint64 on the device. */
int mqa_peak_mfma_bf16(int waves_per_simd, int iters, float* sink, unsigned long long* clocks, void* stream);

/* Streaming read of `bytes` (a multiple of 16 is read; the rest ignored):
 * 4 workgroups of 256 lanes per CU, each reading its own contiguous chunk
 * with 16-byte non-temporal loads, four 1 KB wave loads in flight. */
int mqa_peak_hbm_read(const void* src, size_t bytes, float* sink, void* stream);

/* dst <- src for `bytes` (16-byte units; the rest ignored): reads and
 * writes `bytes` each, non-temporal, each workgroup over its own contiguous
 * chunk. */
int mqa_peak_hbm_copy(const void* src, void* dst, size_t bytes, void* stream);

/* One workgroup of waves_per_cu (1..16) waves per CU; each wave issues
 * iters x 8 ds_read_b128 (1 KB each, conflict-free): bytes read from LDS =
 * CUs x waves_per_cu x iters x 8 x 1024. */
int mqa_peak_lds_read(int waves_per_cu, int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQA_PEAKS_H */
