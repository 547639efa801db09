/* Measurement helper of the H-BitLinear library: a plain streaming read.
 *
 * Not a step of the layer.  It gives the benchmark the time a bare read of a
 * buffer takes on the device, in the same harness as the decode matmul whose
 * cost is dominated by reading its packed ternary weights once (16 MiB at the
 * 7B down-projection shape; the pages tie ternary weights to the memory
 * bandwidth bottleneck: 新智元 article "微软再放LLM量化大招", section
 * 原生4比特盘算).  The read uses the matmul's access shape: each workgroup of
 * 512 threads takes one contiguous 64 KiB chunk, every wave instruction loads
 * 1 KiB contiguously (16 bytes per lane), and all of a thread's loads are
 * issued before any is waited for.
 *
 * Built as its own library, libhbl_calib.so, so the layer's library exports
 * only the layer. */
#ifndef HBL_CALIB_H
#define HBL_CALIB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device address `src` once and writes, for each
 * 64 KiB chunk c (the last one may be shorter), the XOR of its 32-bit words
 * to digest[c] (device, ceil(bytes / 65536) words, caller-owned).
 * src: device, 16-byte aligned; bytes: a positive multiple of 16.
 * Asynchronous on `stream`.  Returns 0 on success, 1 for a null pointer,
 * 2 for a bad size, 4 for a misaligned pointer, 6 if the launch failed;
 * nothing is launched on an error. */
int hbl_calib_stream_read(const void *src, size_t bytes, uint32_t *digest, hipStream_t stream);

/* Every one of `workgroups` workgroups (512 threads each) reads the same
 * `bytes` bytes at `src` once, in the access shape above (1 KiB per wave
 * instruction, eight loads per thread in flight), and writes the XOR of the
 * region's 32-bit words to digest[w] (device, `workgroups` words).  After
 * the first call the region sits in the L2 caches, so this times the L2 to
 * compute-unit path when every CU wants the same bytes -- what the decode
 * matmul asks of it for the activation codes, which every workgroup reads
 * whole.  src: device, 16-byte aligned; bytes: a positive multiple of 16;
 * 1 <= workgroups <= 65536.  Return codes as hbl_calib_stream_read. */
int hbl_calib_broadcast_read(const void *src, size_t bytes, unsigned workgroups, uint32_t *digest,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
