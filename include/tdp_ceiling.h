/*
 * tdp_ceiling.h — memory-system ceilings for the measurement script.
 *
 * Not part of the tiled hot path: these kernels tell how many HBM bytes per
 * second a plain hand-written streaming kernel moves on the GPU at hand, so
 * that the extract and blend rates can be read against an achievable
 * figure as well as against the vendor peak.  Built as its own library,
 * libtdp_ceiling.so.
 */
#ifndef TDP_CEILING_H
#define TDP_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one pass over `bytes` (a multiple of 8192) on `stream` (a
 * hipStream_t, NULL = the null stream) without synchronizing:
 *   mode 0  copy src -> dst, non-temporal loads and stores;
 *   mode 1  copy src -> dst, non-temporal loads, device-scope stores;
 *   mode 2  read src (sink: 4 KB the kernel practically never writes);
 *   mode 3  write dst;
 *   mode 4  gather: dst = src + src[bytes ..] (32-bit lanes; reads 2 *
 *           bytes, writes bytes: the blend's mix);
 *   mode 5  scatter: dst = dst[bytes ..] = src (reads bytes, writes 2 *
 *           bytes: the extract's mix).
 * Device pointers, 16-byte aligned, each holding `bytes` (src in mode 4
 * and dst in mode 5: 2 * bytes; sink: 4096 bytes).
 * Returns 0, -1 for a bad argument (nothing enqueued) or -4 when the launch
 * fails.  The caller owns every buffer. */
int tdp_ceiling_run(int mode, const void* src, void* dst, void* sink, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TDP_CEILING_H */
