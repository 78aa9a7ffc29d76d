// pa_timeline.h -- optional per-workgroup timestamps for the decode kernels
// (internal).  Compiled in only with -DPA_TIMELINE, which build.py --timeline
// uses for the separate diagnostic library libpa_decode_timeline.so; the
// product library libpa_decode.so is built without it and the macros below
// expand to nothing.
//
// Records are four 64-bit words:
//   word 0: kind | XCC id << 4 | linear workgroup id << 8 | HW_ID register << 32
//   words 1-3: start, a mid point, end, read from the 100 MHz constant clock
//              (s_memrealtime; 10 ns ticks, the same clock on every XCD).
// Kinds: 1 Phase 1 / V1 (mid = wave 0 done streaming), 2 Phase 2
// (reduce_split_kernel; mid = the partials have arrived).  One counter numbers
// the records: a Phase-1 workgroup takes its slot when it starts (the atomic's
// latency hides behind the streaming), a Phase-2 workgroup after its end stamp,
// so Phase 2's record adds one atomic round trip to the end of that kernel.
// Records are written through (device-scope relaxed atomic stores), leaving
// no dirty L2 lines for the end of the kernel.
#pragma once

#ifdef PA_TIMELINE
#include <hip/hip_runtime.h>

namespace pa {

constexpr unsigned kTimelineRecords = 1u << 18;
__device__ unsigned long long g_timeline[kTimelineRecords * 4];
__device__ unsigned int g_timeline_count;

__device__ __forceinline__ unsigned long long tl_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ unsigned tl_take_slot() {
    return __hip_atomic_fetch_add(&g_timeline_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void tl_write(unsigned n, unsigned kind, unsigned long long t0,
                                         unsigned long long t1, unsigned long long t2) {
    if (n >= kTimelineRecords) return;
    // HW_ID (hardware register 4, all 32 bits) and XCC_ID (register 20, bits 0-3).
    const unsigned hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
    const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned long long v[4] = {
        (unsigned long long)kind | ((unsigned long long)(xcc & 15u) << 4) |
            ((unsigned long long)(lin & 0xffffffu) << 8) | ((unsigned long long)hw << 32),
        t0, t1, t2};
    for (int i = 0; i < 4; ++i)
        __hip_atomic_store(&g_timeline[4 * (size_t)n + i], v[i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace pa

// Phase 1: slot at the start, record (thread 0) at the end.
#define PA_TL_BEGIN_SLOT()                                   \
    const unsigned long long pa_tl_t0 = ::pa::tl_now();      \
    const unsigned pa_tl_n = threadIdx.x == 0 ? ::pa::tl_take_slot() : 0u
#define PA_TL_MARK(var) const unsigned long long var = ::pa::tl_now()
#define PA_TL_RECORD(kind, t_mid) \
    if (threadIdx.x == 0) ::pa::tl_write(pa_tl_n, kind, pa_tl_t0, t_mid, ::pa::tl_now())
// Phase 2: start stamp only; the slot is taken after the end stamp.
#define PA_TL_BEGIN() const unsigned long long pa_tl_t0 = ::pa::tl_now()
#define PA_TL_RECORD_LATE(kind, t_mid)                                          \
    if (threadIdx.x == 0) {                                                     \
        const unsigned long long pa_tl_t2 = ::pa::tl_now();                     \
        ::pa::tl_write(::pa::tl_take_slot(), kind, pa_tl_t0, t_mid, pa_tl_t2);  \
    }
#else
#define PA_TL_BEGIN_SLOT()
#define PA_TL_MARK(var)
#define PA_TL_RECORD(kind, t_mid)
#define PA_TL_BEGIN()
#define PA_TL_RECORD_LATE(kind, t_mid)
#endif
