/*
 * mla_probe.h - read-stream and issue probes (libmla_probe.so): measurement support for the
 * benchmark, not part of the decode path.
 *
 * The decode step's main loop is bound by the HBM read stream of the latent cache (the
 * pages' point that the cache load is the decode bottleneck: "[ICLR 2025] MLRA…", section 1,
 * and "超越 GQA 的推理革命…MLA…", section 顯存的囚徒).  Next to the published HBM peak
 * the benchmark reports the rate this plain streaming kernel reaches on the same device, the
 * practical ceiling for any kernel that reads each byte once.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Number of uint32 words mla_probe_read writes to `out`. */
size_t mla_probe_out_words(void);

/*
 * Read every byte of `buf` (device, `bytes` long, a multiple of 16, 16-byte aligned) once
 * with 16-byte loads, and write one XOR fold per wave to `out` (device, caller-owned,
 * mla_probe_out_words() words).  Asynchronous on `stream`; time it with events around the
 * call.  Returns 0, 1 for a NULL pointer or a size that is not a multiple of 16, or 6 when
 * the launch fails.  Allocates nothing.
 */
int mla_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

/*
 * The same stream over a paged pool: read every byte of the pages pages[0 .. n_pages-1]
 * (device int32 indices into `pool`, each page `page_bytes` long at pool + index *
 * page_bytes, a multiple of 16) in list order, as a decode reads a shuffled paged cache;
 * mla_probe_out_words() XOR folds go to `out`.  The caller keeps every index inside the
 * pool.  Asynchronous on `stream`.  Returns 0, 1 for a NULL pointer, n_pages < 1 or a page
 * size that is 0, not a multiple of 16 or over 16 MiB, or 6 when the launch fails.
 * Allocates nothing.
 */
int mla_probe_read_pages(const void* pool, size_t page_bytes, const int32_t* pages,
                         int n_pages, uint32_t* out, hipStream_t stream);

/* Number of floats mla_probe_issue writes to `out`. */
size_t mla_probe_issue_out_words(void);

/*
 * Issue probe of one SIMD's matrix core and vector ALU (the rates behind the MFMA-bound
 * kernels' design: how fast MFMA 32x32x16 bf16 chains and v_exp_f32 chains run, alone and
 * side by side).  One workgroup of 8 waves per CU for 256 CUs; `iters` iterations of four
 * independent MFMA chains (matrix waves) or sixteen independent exp2 chains (vector waves).
 * mode: 0 all waves matrix; 1 waves 0-3 matrix and 4-7 vector (one of each per SIMD);
 * 2 waves 0-3 matrix only; 3 waves 4-7 vector only; 4 all waves both, interleaved; 5 all
 * waves vector; 6 waves 0-3 both, interleaved (one wave per SIMD), 4-7 idle.  agpr != 0 keeps
 * the MFMA accumulators in the accumulation registers.
 * `out` (device, caller-owned, mla_probe_issue_out_words() floats) receives meaningless
 * per-lane sums.  Asynchronous on `stream`; time it with events.  Returns 0, 1 for a NULL
 * pointer, a mode outside 0..6 or iters outside 1..2^20, or 6 when the launch fails.
 * Allocates nothing.
 */
int mla_probe_issue(int mode, int agpr, int iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
