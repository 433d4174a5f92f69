/*
 * hbm_probe.h -- measurement helpers for the benchmark (not part of the GEMV
 * library): a read-only HBM streaming probe, which sets the attainable read
 * bandwidth beside the 8 TB/s specification, a one-pass read of a given
 * size (the floor for a call that reads that many bytes), and a plain copy
 * kernel of known size, whose FETCH_SIZE / WRITE_SIZE counter readings
 * calibrate the counters' units.  Each launches one kernel on the given HIP
 * stream and returns 0, or a negative value on bad arguments, or the
 * hipError_t of a failed launch (positive).  Device pointers; the caller owns
 * all memory.
 */
#ifndef HBM_PROBE_H
#define HBM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads nbytes (a positive multiple of 16, buf 16-byte aligned) with 128-bit
 * nontemporal loads; writes one f32 partial sum per workgroup to out[0..blocks). */
int hbm_read_probe(const void *buf, int64_t nbytes, float *out, int blocks, void *hip_stream);

/* Reads nbytes (a positive multiple of 16, at most 2^40, buf 16-byte
 * aligned) in one pass: every wave issues all of its 8 KiB of 128-bit
 * nontemporal loads at once, as the one-shot GEMV kernels do.  Timed over
 * rotating buffers, it gives the shortest launch that merely reads a call's
 * bytes.  out must hold hbm_read_once_blocks(nbytes) floats; nothing is
 * normally written there. */
int hbm_read_once(const void *buf, int64_t nbytes, float *out, void *hip_stream);
int hbm_read_once_blocks(int64_t nbytes);

/* The same read, then one 4-byte store per wave (its sum, reduced over its
 * lanes) to out[wave]: a launch ends only when its stores are acknowledged,
 * so this is the floor for a kernel that reads nbytes and writes a result
 * per wave, as a GEMV does.  out must hold 4 * hbm_read_once_blocks(nbytes)
 * floats. */
int hbm_read_once_store(const void *buf, int64_t nbytes, float *out, void *hip_stream);

/* dst[0..nbytes) = src[0..nbytes) with 128-bit loads and stores; nbytes a
 * positive multiple of 16, both pointers 16-byte aligned, no overlap. */
int hbm_copy(const void *src, void *dst, int64_t nbytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HBM_PROBE_H */
