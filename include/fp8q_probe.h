/*
 * fp8q ceiling probes: plain loops that measure what one MI355X (gfx950)
 * reaches on its matrix cores and on HBM streaming, and its shader clock
 * meanwhile.  They are measurement tools, not part of the FP8 path: the
 * benchmark reports the path's kernels against these measured ceilings next
 * to the published peaks (the pages report only speed ratios on other
 * hardware -- page "Helion in vLLM: FP8 inference of Qwen3", section
 * "Per-kernel performance" -- so the absolute ceilings come from here).
 *
 * Conventions as in fp8q.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t as void*), no allocation, no
 * synchronization; returns 0 on success, 1 for a bad argument, 3 for a
 * misaligned pointer, 7 for a launch failure.
 */
#ifndef FP8Q_PROBE_H
#define FP8Q_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP8Q_PROBE_MFMA_F16 = 0, /* v_mfma_f32_16x16x32_f16 (the exact engine's instruction) */
  FP8Q_PROBE_MFMA_FP8 = 1, /* v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 operands          */
  FP8Q_PROBE_READ = 2,     /* 16-byte loads over a buffer                               */
  FP8Q_PROBE_COPY = 3      /* 16-byte loads and stores                                   */
};

/* Matrix-core loop: `workgroups` workgroups of 256 threads, each wave running
 * `iters` iterations of 8 independent matrix instructions of `kind`.
 *   stamps [workgroups * 4] uint64 (out): per workgroup the shader-clock
 *          counter (s_memtime) before and after its loop, then the 100 MHz
 *          real-time counter (s_memrealtime) before and after;
 *   sink   [workgroups] fp32: never written in practice (keeps the loop).
 * FLOPs per wave and iteration: fp8q_probe_mfma_flops_per_iter(kind). */
int fp8q_probe_mfma(int kind, int64_t iters, int workgroups, uint64_t* stamps, float* sink,
                    void* stream);
int64_t fp8q_probe_mfma_flops_per_iter(int kind);

/* Streaming loop over `bytes` (a multiple of 16) of src with `workgroups`
 * workgroups of 256 threads.  FP8Q_PROBE_READ folds what it reads into one
 * word per thread, written to dst [workgroups * 256] uint32;
 * FP8Q_PROBE_COPY copies src to dst [bytes]. */
int fp8q_probe_stream(int kind, const void* src, void* dst, int64_t bytes, int workgroups,
                      void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8Q_PROBE_H */
