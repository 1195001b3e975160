// Per-wave timelines of the decode kernels, recorded only in the libpa_timeline.so build
// (PA_TIMELINE=1; paged_kv_cache_69_amd/timeline.py reads them). Each wave of a launch writes one
// record: its start, the start of its first tile, the end of its tile loop and its end
// (s_memrealtime, a 100 MHz clock), its XCD / CU / SIMD (the HW_ID and XCC_ID registers) and the
// number of tiles it computed. In the ordinary build every member below compiles to nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef PA_TIMELINE
#define PA_TIMELINE 0
#endif

namespace pa {

constexpr int kTimelineWaves = 16384;  // records per kernel family; waves past this are not recorded
constexpr int kTimelineWords = 8;      // start, first tile, loop end, end, xcc << 32 | hw id, tiles, 0, 0

struct WaveTimeline {
  uint64_t start = 0, first = 0, loop_end = 0;
  int tiles = 0;

  __device__ __forceinline__ void begin() {
    if constexpr (PA_TIMELINE) start = __builtin_amdgcn_s_memrealtime();
  }
  __device__ __forceinline__ void first_tile() {
    if constexpr (PA_TIMELINE) {
      if (first == 0) first = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ __forceinline__ void end_loop(int n) {
    if constexpr (PA_TIMELINE) {
      loop_end = __builtin_amdgcn_s_memrealtime();
      tiles = n;
    }
  }
  // One lane of the wave writes the record with vector stores.
  __device__ __forceinline__ void store(unsigned long long* buf, unsigned idx) {
    if constexpr (PA_TIMELINE) {
      const uint64_t end = __builtin_amdgcn_s_memrealtime();
      const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_ID: wave, SIMD, CU, SE
      const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // XCC_ID
      if ((threadIdx.x & 63) == 0 && idx < (unsigned)kTimelineWaves) {
        unsigned long long* r = buf + (size_t)idx * kTimelineWords;
        r[0] = start;
        r[1] = first;
        r[2] = loop_end;
        r[3] = end;
        r[4] = ((unsigned long long)xcc << 32) | hw;
        r[5] = (unsigned long long)(unsigned)tiles;
      }
    }
  }
};

// Host side of the timeline build: copy a kernel family's records out, or zero them.
int timeline_read_mfma(void* host, size_t bytes);
int timeline_clear_mfma();
int timeline_read_balanced(void* host, size_t bytes);
int timeline_clear_balanced();

}  // namespace pa

#if PA_TIMELINE
// The records of one translation unit's kernels, and the host functions that copy them.
#define PA_TIMELINE_BUFFER(name)                                                                        \
  static __device__ unsigned long long timeline_buf[pa::kTimelineWaves * pa::kTimelineWords];           \
  int pa::timeline_read_##name(void* host, size_t bytes) {                                              \
    if (bytes > sizeof(timeline_buf)) bytes = sizeof(timeline_buf);                                     \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(timeline_buf), bytes, 0, hipMemcpyDeviceToHost);  \
  }                                                                                                     \
  int pa::timeline_clear_##name() {                                                                     \
    void* p = nullptr;                                                                                  \
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(timeline_buf)) != hipSuccess) return -1;                     \
    return (int)hipMemset(p, 0, sizeof(timeline_buf));                                                  \
  }
#define PA_TIMELINE_STORE(tl, idx) (tl).store(timeline_buf, (idx))
#else
#define PA_TIMELINE_BUFFER(name)
#define PA_TIMELINE_STORE(tl, idx) ((void)0)
#endif
