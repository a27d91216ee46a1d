/* Achievable-rate probes (libsa_peaks.so), a measurement companion to
 * libsparse_attn.so.
 *
 * A roofline fraction is quoted twice: against the datasheet peak (HBM3E
 * 8 TB/s, dense bf16 matrix 2.5 PFLOP/s) and against what these kernels
 * reach on the machine they run on; the LDS read rate has no datasheet
 * figure here and sets how far the attention kernels' operand reads can
 * keep up with their products.  No function is on the attention path.
 *
 * All launch asynchronously on `stream` (a hipStream_t, NULL = the default
 * stream); the caller times them with events on that stream.  All return a
 * hipError_t value as int: 0 on success, hipErrorInvalidValue (1) for a NULL
 * pointer, a misaligned buffer or iters < 1, otherwise the launch error.
 * Nothing is allocated, freed or synchronised.
 */
#ifndef SA_PEAKS_H
#define SA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_PEAKS_EXPORT __attribute__((visibility("default")))

/* Read `bytes` (rounded down to a multiple of 16 KiB, written to *bytes_read)
 * of the device buffer `buf` (16-byte aligned) once, with 16-byte
 * non-temporal loads from eight 256-thread workgroups per compute unit.  Use
 * a buffer several times the 256 MB last-level cache.  `sink` is a device
 * buffer of at least 1 KiB that the kernel may write (it never does for real
 * data; the store only keeps the loads alive). */
SA_PEAKS_EXPORT int sa_peak_read(const void* buf, size_t bytes, void* sink, void* stream,
                                 size_t* bytes_read);

/* Run `iters` rounds of four independent 32x32x16 bf16 matrix-core products
 * per wave on eight 256-thread workgroups per compute unit; *flops receives
 * the algorithmic flop count of the launch (32*32*16*2 per product).  `sink`
 * as above. */
SA_PEAKS_EXPORT int sa_peak_mfma_bf16(int iters, void* sink, void* stream, double* flops);

/* Run `iters` rounds of 32 products per wave (eight operand pairs of random
 * bf16 values in [-2, 2), taken in turn, on four independent 32x32x16
 * accumulator chains) on two 256-thread workgroups per compute unit;
 * *flops as above.  Products over changing data draw more power than the
 * one-pair loop above, and the chip's clock under load follows its power:
 * this is the product rate for data like an attention kernel's. */
SA_PEAKS_EXPORT int sa_peak_mfma_bf16_data(int iters, void* sink, void* stream, double* flops);

/* Run `iters` rounds of sixteen 16-byte LDS reads per lane (ds_read_b128,
 * bank-conflict free, all in flight together) on four 256-thread workgroups
 * per compute unit, each reading its own 32 KB of LDS; *bytes receives the
 * bytes read by the launch.  Divide by the time and the compute unit count
 * for the per-CU rate.  `sink` as above. */
SA_PEAKS_EXPORT int sa_peak_lds_read(int iters, void* sink, void* stream, double* bytes);

#ifdef __cplusplus
}
#endif

#endif /* SA_PEAKS_H */
