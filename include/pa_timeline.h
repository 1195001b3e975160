/*
 * pa_timeline.h: the two extra entry points of libpa_timeline.so, a build of the decode library
 * (every pa.h entry point, the same kernels) whose decode kernels also record one timeline entry
 * per wave of their latest launch: the wave's start, the start of its first tile, the end of its
 * tile loop and its end (the GPU's 100 MHz s_memrealtime clock), its XCD / CU / SIMD and the tiles
 * it computed. It is a measurement build (python -m paged_kv_cache_69_amd._build --timeline;
 * paged_kv_cache_69_amd/timeline.py reads the records); libpa.so does not export these.
 */
#ifndef PA_TIMELINE_H_
#define PA_TIMELINE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families with their own record buffers. */
enum { PA_TIMELINE_MFMA = 0, PA_TIMELINE_BALANCED = 1 };

/* Record layout: 8 uint64 per wave, indexed by blockIdx.x * waves_per_workgroup + wave: start,
 * first tile (0: none), loop end (0: none), end, (XCC_ID << 32) | HW_ID, tiles, 0, 0. At most
 * PA_TIMELINE_WAVES waves per family; an entry whose start is 0 was not written. */
#define PA_TIMELINE_WAVES 16384

/* Copy up to `bytes` bytes of a family's records into host memory `host` (synchronous). 0 on
 * success, -1 for an unknown family, else the HIP error code. */
int pa_timeline_read(int32_t family, void* host, size_t bytes);

/* Zero every family's records (synchronous). 0 on success. */
int pa_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_TIMELINE_H_ */
