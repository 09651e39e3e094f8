/*
 * sparse_mla_measure.h - measurement entry point of the sparse-MLA library.
 *
 * For benchmarks that measure the gather roofline of the fp8_ds_mla row
 * format: not part of the attention computation.
 */
#ifndef SPARSE_MLA_MEASURE_H
#define SPARSE_MLA_MEASURE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

/* The library exports its entry points and nothing else. */
#ifndef SMLA_API
#define SMLA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * smla_gather_rows_probe - read the rows an attention call would gather, and
 * nothing else.
 *
 * Reads the bytes of every listed cache row that sparse_mla_attn gathers for
 * it -- the first 528 bytes (rope_dim 0: codes and scales) or all 656 bytes
 * (rope_dim 64) -- with plain 16-byte loads, eight in flight per lane, one
 * 512-thread workgroup per CU, and folds the loaded words by XOR into *sink
 * (so that the loads cannot be dropped).  The time it takes for a list of rows
 * is what the memory system delivers for that list with no arithmetic; the
 * attention kernel's time on the same rows is compared with it.  Entries
 * outside [0, num_slots) are skipped.
 *
 * kv_cache  uint8 [num_slots][656], 16-byte aligned; num_slots >= 1.
 * rope_dim  64 or 0.
 * slots     int32 [n] slot numbers (e.g. the valid entries of a top-k buffer).
 * n         0 <= n <= 2,097,152 (256 workgroups of at most 8,192 rows).
 * sink      one uint32 of device memory, XOR-updated (its value is meaningless).
 * Errors as for the other calls: SMLA_EINVAL for bad arguments, SMLA_EUNSUPPORTED
 * for n beyond the limit, SMLA_ELAUNCH if the launch fails.
 */
SMLA_API int smla_gather_rows_probe(const void* kv_cache, int64_t num_slots, int rope_dim,
                           const int32_t* slots, int64_t n, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_MEASURE_H */
