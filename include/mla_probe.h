/*
 * mla_probe.h - read-stream probe (libmla_probe.so): measurement support for the decode
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

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
