/*
 * ckks_probe.h -- device calibration of libckks_mi355x.so (measurement aid).
 *
 * The benchmark reports each kernel against the measured ceilings of this
 * chip rather than against derived per-operation prices: the issue rate of
 * the integer instructions the kernels are built from, the rate of the
 * library's own 64-bit modular primitives (the "modmul-class" operation the
 * key-switch work is counted in) and the device copy rate at several sizes
 * (HBM, or Infinity Cache when the buffers fit in it).
 */
#ifndef CKKS_MI355X_PROBE_H
#define CKKS_MI355X_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Comma-separated names of the probes into buf[len] (NUL-terminated):
 * single instructions ("v_mul_lo_u32", "v_mad_u64_u32", ...), modular
 * primitives ("shoup", "shoup_lazy", "shoup_split", "mont_lazy", "mac128",
 * "split_mac", "butterfly_ct", "butterfly_gs") and "copy".
 * CKKS_EINVAL if buf is NULL or too small. */
int ckks_probe_list(char* buf, int len);

/* Runs probe `what` on HIP device hip_device (synchronously, on the null
 * stream; the device is otherwise idle) and writes its rate to *rate:
 *   ALU probes  lane-operations per second (one instruction, one modular
 *               product, one multiply-accumulate or one butterfly per lane),
 *               median of 9 timed launches of 8 waves per SIMD, each lane
 *               running 16 independent chains;
 *   "copy"      bytes read plus bytes written per second of a device copy of
 *               copy_bytes (a positive multiple of 4096; two buffers of that
 *               size are allocated and freed), median of 15 copies; one
 *               16-byte word per thread and one 4 KiB block per workgroup.
 * *ms (optional) receives the median launch time.  copy_bytes is ignored by
 * the ALU probes.  Returns CKKS_OK, CKKS_EINVAL (unknown probe, bad size),
 * CKKS_ENOMEM or CKKS_EHIP. */
int ckks_probe_rate(int hip_device, const char* what, uint64_t copy_bytes, double* rate, double* ms);

#ifdef __cplusplus
}
#endif

#endif /* CKKS_MI355X_PROBE_H */
