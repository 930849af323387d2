/*
 * nq_measure.h -- measurement aid of the MI355X (gfx950) packed-weight
 * decoder library: a streaming kernel with a decode's memory traffic and no
 * arithmetic, whose throughput is the practical HBM ceiling for a decode that
 * reads and writes the same byte counts.  It belongs to no page's operation;
 * it puts a measured bound beside the decode's throughput.
 */
#ifndef NQ_MEASURE_H
#define NQ_MEASURE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flags of nq_measure_stream. */
enum { NQ_STREAM_NT_LOAD = 1, NQ_STREAM_NT_STORE = 2 };

/* Read src_bytes from src and write dst_bytes to dst, asynchronously on
 * `stream`.  The output is cut into tiles of 256 threads x C 16-byte chunks,
 * C = chunks_per_thread (1, 2, 4 or 8; a tile is the output of one 16-bit
 * decode tile of C units per thread); tile t reads its proportional share of
 * the source, 16-byte chunks [t*ns/T, (t+1)*ns/T) of T tiles, and each
 * thread stores the XOR of its loaded chunks (further XORed with the
 * store's index within the thread) to its C output chunks.  Loads are
 * non-temporal with NQ_STREAM_NT_LOAD, stores with NQ_STREAM_NT_STORE.  The
 * written bytes carry no meaning.
 *
 * Requirements: src and dst non-NULL (NQ_ERR_NULL_ARG) and 16-byte aligned
 * (NQ_ERR_MISALIGNED); 0 < dst_bytes, src_bytes <= dst_bytes, both multiples
 * of 16, chunks_per_thread one of 1, 2, 4, 8 and no other flag bits
 * (NQ_ERR_BAD_DIM); dst_bytes <= 2^40 (NQ_ERR_OVERFLOW).  NQ_ERR_HIP if the
 * launch failed.  The buffers must not overlap; the caller owns them. */
int nq_measure_stream(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes, int32_t chunks_per_thread,
                      int32_t flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
