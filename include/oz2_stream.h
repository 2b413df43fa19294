/* oz2_stream.h -- HBM stream kernels of known size, the measured bandwidth
 * ceilings against which the memory-bound phases of oz2 are judged (the Arc
 * page, "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc
 * GPUs: Ozaki Scheme II on the Xe2 Architecture", Sec. 3 Table 1, measures
 * its own copy rate with random data for the same purpose).  A measurement
 * aid built into liboz2_stream.so; not part of the method. */
#ifndef OZ2_STREAM_H
#define OZ2_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    OZ2_STREAM_READ = 0,   /* load every 16-byte word of src once */
    OZ2_STREAM_WRITE = 1,  /* store every 16-byte word of dst once (index-dependent values) */
    OZ2_STREAM_COPY = 2    /* dst <- src */
};

/* Enqueue one stream of `bytes` (a positive multiple of 16) on `stream` (a
 * hipStream_t, NULL for the null stream): `blocks` blocks of 256 threads in
 * a grid-stride loop, `unroll` in {1, 2, 4, 8} 16-byte words per thread per
 * trip with their loads issued before any use, nontemporal != 0 for
 * nontemporal loads and stores.  src and dst are DEVICE pointers owned by
 * the caller: src holds `bytes` (READ, COPY); dst holds `bytes` (WRITE,
 * COPY) or, for READ, blocks * 4096 bytes that receive one folded word per
 * thread.  Returns 0, -i for an invalid argument i, or 2 when the launch
 * fails.  Asynchronous: time it with events on the same stream. */
int oz2_stream_run(int kind, const void* src, void* dst, int64_t bytes, int blocks, int unroll,
                   int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OZ2_STREAM_H */
