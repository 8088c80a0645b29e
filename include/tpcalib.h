/*
 * tpcalib.h -- C ABI of libtpcalib: a measurement helper, not part of the
 * method.  It measures the bf16 MFMA rate a gfx950 GPU sustains when nothing
 * but matrix instructions run, which is the practical ceiling the GEMM
 * kernels of libtpshard are measured against (the nominal peak assumes the
 * 2.4 GHz clock at every MFMA density; under a board power limit the clock
 * drops with the power the matrix cores draw, which depends on the data).
 */
#ifndef TPCALIB_H
#define TPCALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TPC_API
#define TPC_API __attribute__((visibility("default")))
#endif

/*
 * Launches one workgroup of 4 wave64s per CU (`cus` workgroups).  Each wave
 * loads its operand fragments (bf16, 8 per lane) from `src` once and then
 * issues matrix instructions into independent accumulator blocks held in the
 * 256 accumulator registers, cycling through its fragments so that
 * consecutive instructions see different operands; no memory traffic and no
 * LDS inside the loop.
 *   shape 32: v_mfma_f32_32x32x16_bf16, 16 blocks, 16 fragments per wave
 *             (wave w reads 16 KiB at src + (w % 4) * 16 KiB), 32
 *             instructions (1048576 FLOP) per iteration;
 *   shape 16: v_mfma_f32_16x16x32_bf16, 32 blocks, 24 fragments per wave
 *             (24 KiB at src + (w % 4) * 24 KiB), 64 instructions
 *             (1048576 FLOP) per iteration.
 * src: >= 96 KiB, 16-byte aligned, device.  out: fp32 [cus * 256] (one
 * checksum per thread, device) so the work cannot be elided.  FLOPs of one
 * call: cus * 4 * iters * (FLOP per iteration).  Returns 0, -1 for a NULL
 * pointer, iters < 1, cus < 1 or another shape (nothing launched), else the
 * hipError_t of the launch.  Asynchronous on `stream` (NULL = default).
 */
TPC_API int tpc_mfma_loop(const void* src, float* out, int cus, int iters, int shape, void* stream);

/*
 * Shader clock probe: `blocks` workgroups of one wave64 each read the shader
 * cycle counter and the 100 MHz real-time counter, run `spin` dependent
 * integer steps, and read both again.  out: device uint64 [2 * blocks]:
 * (cycles, real-time ticks) elapsed per workgroup; cycles / ticks * 100 is
 * the clock in MHz.  Returns 0, -1 for a NULL pointer, blocks < 1 or
 * spin < 1 (nothing launched), else the hipError_t of the launch.
 * Asynchronous on `stream` (NULL = default).
 */
TPC_API int tpc_clock_probe(unsigned long long* out, int blocks, int spin, void* stream);

/*
 * LDS read-rate probe: `cus` workgroups of `waves` (1..16) wave64s, each
 * reading its workgroup's 64 KiB LDS array `iters` times 8 reads (8 in
 * flight, the address moving every iteration), in one pattern:
 *   kind 0: ds_read_b128, 16 bytes per lane, 1 KiB of consecutive bytes;
 *   kind 1: ds_read_b64_tr_b16, 8 bytes per lane, 512 consecutive bytes;
 *   kind 2: ds_read_b64_tr_b16 as the attention kernels read the columns of
 *           a 256-byte-row tile (chunk c of row r at c ^ (4 (r % 4) +
 *           (r / 4) % 4)).
 * Bytes read per workgroup: waves * 64 * (16 or 8) * 8 * iters.  cycles:
 * device uint64 [cus], shader cycles of each workgroup's read loop; out:
 * device uint32 [cus * 64 * waves] checksums.  Returns 0, -1 for a NULL
 * pointer or an argument out of range (nothing launched), else the
 * hipError_t of the launch.  Asynchronous on `stream` (NULL = default).
 */
TPC_API int tpc_lds_read_rate(unsigned* out, unsigned long long* cycles, int cus, int waves, int iters, int kind,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TPCALIB_H */
