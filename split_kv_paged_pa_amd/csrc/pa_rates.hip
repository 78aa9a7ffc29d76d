// pa_rates.hip -- instruction-rate probe (measurement only; part of
// libpa_probe.so, not of the attention library).  Each wave runs one kind of
// instruction stream for `iters` rounds and records its elapsed shader clock
// (s_memtime) and constant 100 MHz clock (s_memrealtime); the ratio gives the
// clock frequency, the first the cycles per instruction.  Kinds:
//   0: v_exp_f32 x 8 independent chains      1: v_fma_f32 x 8 chains
//   2: v_mfma_f32_16x16x32_bf16 x 8 accumulators
//   3: 8 of those MFMAs, each followed by 3 independent v_fma_f32
//   4: ds_read_b128 x 8 (lane l reads bytes 16 l .. 16 l + 15 of its wave's
//      8 KiB window, conflict-free), then a wait for all of them.
// Waves 0-3 of a workgroup run kind `lo`, waves 4-7 kind `hi`; with 512 threads
// waves w and w + 4 share a SIMD.  All instruction streams are written as asm
// so that the counts are exact; the LDS reads wait in the same asm block.
//
// A second kernel reads LDS with a caller-given 16-byte offset per lane (the
// same 64 offsets in every wave), to measure which lane patterns of a 128-bit
// LDS read conflict: its clocks per read, and the LDS bank-conflict counter of
// its dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__device__ __forceinline__ float rate_work(int iters, float seed, const char *lds_window) {
    float a0 = seed, a1 = seed + 1, a2 = seed + 2, a3 = seed + 3, a4 = seed + 4, a5 = seed + 5,
          a6 = seed + 6, a7 = seed + 7;
    if constexpr (KIND == 0) {
        for (int i = 0; i < iters; ++i)
            asm volatile("v_exp_f32 %0, %0\n v_exp_f32 %1, %1\n v_exp_f32 %2, %2\n v_exp_f32 %3, %3\n"
                         "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n v_exp_f32 %6, %6\n v_exp_f32 %7, %7"
                         : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
    } else if constexpr (KIND == 1) {
        for (int i = 0; i < iters; ++i)
            asm volatile("v_fma_f32 %0, %0, %0, %0\n v_fma_f32 %1, %1, %1, %1\n"
                         "v_fma_f32 %2, %2, %2, %2\n v_fma_f32 %3, %3, %3, %3\n"
                         "v_fma_f32 %4, %4, %4, %4\n v_fma_f32 %5, %5, %5, %5\n"
                         "v_fma_f32 %6, %6, %6, %6\n v_fma_f32 %7, %7, %7, %7"
                         : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
    } else if constexpr (KIND == 2 || KIND == 3) {
        f32x4 c0 = {seed, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
        bf16x8 x;
        for (int j = 0; j < 8; ++j) x[j] = (__bf16)(seed * j);
        for (int i = 0; i < iters; ++i) {
            if constexpr (KIND == 2) {
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %8, %8, %0\n v_mfma_f32_16x16x32_bf16 %1, %8, %8, %1\n"
                             "v_mfma_f32_16x16x32_bf16 %2, %8, %8, %2\n v_mfma_f32_16x16x32_bf16 %3, %8, %8, %3\n"
                             "v_mfma_f32_16x16x32_bf16 %4, %8, %8, %4\n v_mfma_f32_16x16x32_bf16 %5, %8, %8, %5\n"
                             "v_mfma_f32_16x16x32_bf16 %6, %8, %8, %6\n v_mfma_f32_16x16x32_bf16 %7, %8, %8, %7"
                             : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
                             : "v"(x));
            } else {
                asm volatile(
                    "v_mfma_f32_16x16x32_bf16 %0, %14, %14, %0\n v_fma_f32 %8, %8, %8, %8\n v_fma_f32 %9, %9, %9, %9\n v_fma_f32 %10, %10, %10, %10\n"
                    "v_mfma_f32_16x16x32_bf16 %1, %14, %14, %1\n v_fma_f32 %11, %11, %11, %11\n v_fma_f32 %12, %12, %12, %12\n v_fma_f32 %13, %13, %13, %13\n"
                    "v_mfma_f32_16x16x32_bf16 %2, %14, %14, %2\n v_fma_f32 %8, %8, %8, %8\n v_fma_f32 %9, %9, %9, %9\n v_fma_f32 %10, %10, %10, %10\n"
                    "v_mfma_f32_16x16x32_bf16 %3, %14, %14, %3\n v_fma_f32 %11, %11, %11, %11\n v_fma_f32 %12, %12, %12, %12\n v_fma_f32 %13, %13, %13, %13\n"
                    "v_mfma_f32_16x16x32_bf16 %4, %14, %14, %4\n v_fma_f32 %8, %8, %8, %8\n v_fma_f32 %9, %9, %9, %9\n v_fma_f32 %10, %10, %10, %10\n"
                    "v_mfma_f32_16x16x32_bf16 %5, %14, %14, %5\n v_fma_f32 %11, %11, %11, %11\n v_fma_f32 %12, %12, %12, %12\n v_fma_f32 %13, %13, %13, %13\n"
                    "v_mfma_f32_16x16x32_bf16 %6, %14, %14, %6\n v_fma_f32 %8, %8, %8, %8\n v_fma_f32 %9, %9, %9, %9\n v_fma_f32 %10, %10, %10, %10\n"
                    "v_mfma_f32_16x16x32_bf16 %7, %14, %14, %7\n v_fma_f32 %11, %11, %11, %11\n v_fma_f32 %12, %12, %12, %12\n v_fma_f32 %13, %13, %13, %13"
                    : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7),
                      "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5)
                    : "v"(x));
            }
        }
        a0 += c0[0] + c1[1] + c2[2] + c3[3] + c4[0] + c5[1] + c6[2] + c7[3];
    } else if constexpr (KIND == 4) {
        const unsigned base = (unsigned)(uintptr_t)(lds_window + (threadIdx.x & 63) * 16);  // LDS byte offset
        uint32_t acc = 0;
        for (int i = 0; i < iters; ++i) {
            uint4 v0, v1, v2, v3, v4, v5, v6, v7;
            asm volatile(
                "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:1024\n ds_read_b128 %2, %8 offset:2048\n"
                "ds_read_b128 %3, %8 offset:3072\n ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %8 offset:5120\n"
                "ds_read_b128 %6, %8 offset:6144\n ds_read_b128 %7, %8 offset:7168\n s_waitcnt lgkmcnt(0)"
                : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
                : "v"(base));
            acc ^= v0.x ^ v1.y ^ v2.z ^ v3.w ^ v4.x ^ v5.y ^ v6.z ^ v7.w;
        }
        a0 += (float)acc;
    }
    return a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

// One record per wave: {shader clocks, 100 MHz clocks, result sink}.
template <int LO, int HI>
__global__ __launch_bounds__(512) void rate_kernel(unsigned long long *__restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) char lds[4 * 8192];
    for (int i = threadIdx.x; i < 4 * 8192 / 4; i += blockDim.x) reinterpret_cast<uint32_t *>(lds)[i] = i;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const char *window = lds + (wave & 3) * 8192;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const float sink = (wave & 4) ? rate_work<HI>(iters, 0.5f, window) : rate_work<LO>(iters, 0.5f, window);
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
        const unsigned w = blockIdx.x * (blockDim.x / 64) + wave;
        out[3 * w + 0] = t1 - t0;
        out[3 * w + 1] = r1 - r0;
        out[3 * w + 2] = __float_as_uint(sink);
    }
}

template <int LO, int HI>
int launch_rate(void *out, int blocks, int threads, int iters, hipStream_t st) {
    hipLaunchKernelGGL((rate_kernel<LO, HI>), dim3(blocks), dim3(threads), 0, st,
                       static_cast<unsigned long long *>(out), iters);
    return (int)hipGetLastError();
}

constexpr int kPatternLds = 32768;              // bytes of LDS the pattern kernel reads
constexpr int kPatternSpan = 7 * 1024 + 16;      // bytes one lane's 8 reads cover past its offset
constexpr int kPatternMaxOffset = kPatternLds - kPatternSpan;

// 256 threads (one wave per SIMD); per round each wave issues 8 ds_read_b128 at
// its lane's offset + 1024 k, then waits.  Offsets are clamped into the array
// and rounded down to 16 bytes, so every read stays inside it.
__global__ __launch_bounds__(256) void lds_pattern_kernel(const int *__restrict__ offsets,
                                                         unsigned long long *__restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) char lds[kPatternLds];
    for (int i = threadIdx.x; i < kPatternLds / 4; i += blockDim.x) reinterpret_cast<uint32_t *>(lds)[i] = i;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const int off = min(max(offsets[threadIdx.x & 63], 0), kPatternMaxOffset) & ~15;
    const unsigned base = (unsigned)(uintptr_t)(lds + off);
    uint32_t acc = 0;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
        uint4 v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:1024\n ds_read_b128 %2, %8 offset:2048\n"
            "ds_read_b128 %3, %8 offset:3072\n ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %8 offset:5120\n"
            "ds_read_b128 %6, %8 offset:6144\n ds_read_b128 %7, %8 offset:7168\n s_waitcnt lgkmcnt(0)"
            : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
            : "v"(base));
        acc ^= v0.x ^ v1.y ^ v2.z ^ v3.w ^ v4.x ^ v5.y ^ v6.z ^ v7.w;
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    if ((threadIdx.x & 63) == 0) {
        const unsigned w = blockIdx.x * 4 + wave;
        out[2 * w + 0] = t1 - t0;
        out[2 * w + 1] = acc;
    }
}

}  // namespace

// offsets: 64 ints in device memory, the byte offset each lane reads at (clamped
// to [0, 32768 - 7 * 1024 - 16], rounded down to 16).  out: 2 * 4 * blocks u64
// records {shader clocks, sink} per wave.  Returns 0, or -1 for bad arguments.
extern "C" int pa_probe_lds_pattern(const void *offsets, void *out, int blocks, int iters, void *stream) {
    if (offsets == nullptr || out == nullptr || blocks <= 0 || iters <= 0) return -1;
    hipLaunchKernelGGL(lds_pattern_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const int *>(offsets), static_cast<unsigned long long *>(out), iters);
    return (int)hipGetLastError();
}

// out: 3 * blocks * threads / 64 u64 records.  threads 256 or 512; (lo, hi) one of
// the pairs below, else -1.
extern "C" int pa_probe_rates(int lo, int hi, void *out, int blocks, int threads, int iters, void *stream) {
    if (out == nullptr || blocks <= 0 || (threads != 256 && threads != 512) || iters <= 0) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int key = lo * 8 + hi;
    switch (key) {
        case 0 * 8 + 0: return launch_rate<0, 0>(out, blocks, threads, iters, st);
        case 1 * 8 + 1: return launch_rate<1, 1>(out, blocks, threads, iters, st);
        case 2 * 8 + 2: return launch_rate<2, 2>(out, blocks, threads, iters, st);
        case 3 * 8 + 3: return launch_rate<3, 3>(out, blocks, threads, iters, st);
        case 4 * 8 + 4: return launch_rate<4, 4>(out, blocks, threads, iters, st);
        case 2 * 8 + 1: return launch_rate<2, 1>(out, blocks, threads, iters, st);
        case 2 * 8 + 0: return launch_rate<2, 0>(out, blocks, threads, iters, st);
        case 2 * 8 + 4: return launch_rate<2, 4>(out, blocks, threads, iters, st);
        default: return -1;
    }
}
