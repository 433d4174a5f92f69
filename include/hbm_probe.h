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
 * per wave, as a GEMV does.  Several launch shapes, so that the floor a call
 * is measured against is the best of them:
 *   shape 0: one pass, 4-wave workgroups, 8 loads of 16 bytes per lane;
 *   shape 1: one pass, 16-wave workgroups, 4 loads per lane;
 *   shape 2: a resident grid (2 workgroups per compute unit) of 16-wave
 *            workgroups whose waves walk the buffer 4 loads per lane at a
 *            time.
 * nbytes and buf as for hbm_read_once; out must hold
 * hbm_read_floor_out_floats(nbytes, shape) floats.  Returns -1 on bad
 * arguments (also for shape outside 0..hbm_read_floor_shapes()-1). */
int hbm_read_floor_shapes(void);
int64_t hbm_read_floor_out_floats(int64_t nbytes, int shape);
int hbm_read_floor(const void *buf, int64_t nbytes, float *out, int shape, void *hip_stream);

/* The one-column GEMV's arithmetic alone for an N x K call of format wfmt
 * (a GEMV_W_* value): every row's ceil(K / E / 64) chunks per lane of 16
 * bytes decoded and multiplied into f32 sums with the library's own decoders
 * (E values per chunk), then reduced over the wave, one row per wave in
 * 8-wave workgroups, on words made in registers: no weight byte is read.
 * Its launch time is the floor the vector ALUs set for that call.  x: at
 * least 64 floats; out: N floats (row sums of the synthetic words).
 * Returns -1 on bad arguments. */
int gemv_valu_floor(int wfmt, int64_t N, int64_t K, const float *x, float *out, void *hip_stream);

/* dst[0..nbytes) = src[0..nbytes) with 128-bit loads and stores; nbytes a
 * positive multiple of 16, both pointers 16-byte aligned, no overlap. */
int hbm_copy(const void *src, void *dst, int64_t nbytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HBM_PROBE_H */
