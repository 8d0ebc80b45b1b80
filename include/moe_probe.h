/* moe_probe.h -- the HBM read probe of libmoe_probe.so, a measurement aid
 * kept apart from the MoE interface in moe.h.
 *
 * It gives the achievable HBM read rate that the measurements report beside
 * the 8 TB/s specification, read two ways, both with the non-temporal hint:
 * by LDS DMA (one block per compute unit streams 1 MiB pieces of a buffer
 * into LDS, 32 KiB per step in a three-stage ring -- the access pattern of
 * the grouped GEMM's streamed weights, without MFMAs) and by 16-byte register
 * loads (the pattern of its register-path weight loads).  A third form reads
 * in the GEMM's own weight pattern and writes an output burst after every
 * 256-row tile, as the GEMM's units store their output tiles: it gives the
 * achievable read rate when a share of the traffic is writes.
 */
#ifndef MOE_PROBE_H_
#define MOE_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the `bytes` bytes at device address `buf` once, enqueued on `stream`
 * (a hipStream_t as void*; NULL = the default stream) without synchronising.
 *   buf    device memory, 16-byte aligned, owned by the caller
 *   bytes  a positive multiple of 1 MiB
 *   sink   device memory of at least one uint32_t per compute unit; the kernel
 *          writes it only if a folded checksum of the data hits one fixed value
 * Returns 0 when the launch was enqueued, 1 on unusable sizes, a NULL pointer
 * or a failed launch (nothing is enqueued then). */
int moe_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* As moe_probe_hbm_read, with non-temporal register loads: eight blocks of 256
 * threads per compute unit, each thread with eight 16-byte loads in flight.
 * Same arguments, ownership and return values; `buf` must be 16-byte aligned
 * (else 1, nothing enqueued). */
int moe_probe_hbm_read_nt(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* A weight stream with writes, in the grouped GEMM's pattern: `buf` is read
 * as pieces of 256 rows of `row_bytes` each (a 256-row weight tile), 128 bytes
 * of every row per 32 KiB step, with the same LDS DMA, ring and non-temporal
 * hint as moe_probe_hbm_read; piece p starts at column p mod (row_bytes / 128)
 * and wraps round.  After each piece, `out_per_piece` bytes are written to
 * `out` with 16-byte non-temporal stores (piece p's at out + p * out_per_piece).
 *   buf            device memory, owned by the caller
 *   bytes          a positive multiple of 256 * row_bytes
 *   row_bytes      a positive multiple of 128, at most 1 MiB
 *   out            device memory of (bytes / (256 * row_bytes)) * out_per_piece
 *                  bytes, 16-byte aligned, owned by the caller; its contents
 *                  are left undefined
 *   out_per_piece  a positive multiple of 16, at most 256 * row_bytes
 *   sink, stream   as for moe_probe_hbm_read
 * Returns 0 when the launch was enqueued, 1 on unusable sizes, a NULL or
 * misaligned pointer or a failed launch (nothing is enqueued then). */
int moe_probe_hbm_read_write(const void* buf, int64_t bytes, int64_t row_bytes, void* out, int64_t out_per_piece,
                             uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H_ */
