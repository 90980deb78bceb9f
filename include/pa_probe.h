/*
 * pa_probe.h -- HBM read probe of the paged-attention library (measurement).
 *
 * Paged decode is bound by reading the KV cache (page "vLLM框架是怎么做推理加速的",
 * section 3: the decode phase is dominated by KV-cache reads), so its speed
 * follows HBM bandwidth (page "字节跳动 AI Infra (2)", third question,
 * layer-4 table, the HBM3E row).  This probe measures the read rate a kernel
 * actually reaches on the current GPU for the two access patterns that
 * matter: one sequential pass over a buffer, and whole tiles read in a
 * scattered order, the shape of a block-table gather (each (block, kv head)
 * tile is contiguous, consecutive tiles are not).  A sequential pass with
 * ordinary loads over a buffer larger than the L2s and the Infinity Cache
 * also evicts them (the flush between timed benchmark steps).
 *
 * Conventions as in pa.h: device pointers, launched on `stream`, nothing
 * allocated, no synchronisation, PA_OK means "valid and launched".
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_PROBE_SEQ = 0,      /* every 16 bytes of buf once, in address order, ordinary loads */
  PA_PROBE_SEQ_NT = 1,   /* the same with non-temporal loads */
  PA_PROBE_TILES = 2,    /* whole tiles of tile_bytes in a scattered order, ordinary loads */
  PA_PROBE_TILES_NT = 3  /* the same with non-temporal loads */
} pa_probe_mode;

/*
 * pa_probe_read -- read a device buffer once and discard it.
 *
 *   buf         device memory, 16-byte aligned, `bytes` readable bytes
 *   bytes       > 0, a multiple of 16
 *   mode        a pa_probe_mode value
 *   tile_bytes  tile modes: a multiple of 16, 16 <= tile_bytes <= bytes.  The
 *               pass reads the first ntiles tiles of buf, ntiles the largest
 *               power of two with ntiles * tile_bytes <= bytes, each exactly
 *               once, tile t of the pass being tile (t * c1 + c0) mod ntiles
 *               (c1 odd: a bijection).  Ignored by the sequential modes.
 *   sink        device uint32, 4-byte aligned: written only if the XOR of a
 *               thread's words equals a fixed constant (practically never),
 *               which keeps every load live.
 * Bytes read: `bytes` (rounded down to 16) for the sequential modes,
 * ntiles * tile_bytes for the tile modes.  Errors: PA_ERR_NULL_PTR,
 * PA_ERR_BAD_SHAPE (sizes), PA_ERR_UNSUPPORTED (mode), PA_ERR_MISALIGNED.
 */
pa_status pa_probe_read(const void *buf, size_t bytes, int32_t mode, int32_t tile_bytes, uint32_t *sink,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
