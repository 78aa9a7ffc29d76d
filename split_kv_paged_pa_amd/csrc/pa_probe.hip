// pa_probe.hip -- HBM read-bandwidth probe for gfx950 (measurement only; not part
// of the attention ABI).  It reads memory with the same access shape as the
// decode kernels -- 16-byte non-temporal loads, one chunk of `chunk_bytes` per
// wave at a time, several chunks in flight per wave -- and does no arithmetic
// beyond folding the loaded words into one value per thread, so its bandwidth
// is the ceiling the attention kernels can approach for the same chunk order.
//
//   pa_probe_read(base, chunk_ids, num_chunks, chunk_bytes, waves_per_group,
//                 num_groups, shape, sink, stream)
// Chunk k is at base + chunk_ids[k] * chunk_bytes (chunk_ids NULL: chunk k).
// shape 0: each load instruction of a wave covers 1 KiB of contiguous bytes.
// shape 1: a 4 KiB chunk seen as 16 rows of 256 bytes (a token-major block):
//          lane l reads 16 bytes of row l % 16 at byte 16 * (l / 16) + 64 * c of
//          the row, so an instruction covers 64 bytes of each row.  (The decode
//          kernels' split cache layout reads as shape 0: 1 KiB of keys, 512 B of
//          values contiguous per instruction.)
// The chunks are split evenly over num_groups workgroups of waves_per_group
// waves; sink receives one uint32 per thread (num_groups * waves_per_group * 64).
// Returns 0 on success, 1 for invalid arguments, 2 for a failed launch.
//
//   pa_probe_read_xcd(..., sink, times, stream)
// The same with shape 0, plus three uint64 per workgroup in `times`: the 100 MHz
// constant clock when its wave 0 starts and when it has folded its last chunk,
// and the XCC (XCD) id it ran on -- to compare the XCDs' read rates.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kInFlight = 4;  // chunks in flight per wave

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16-byte non-temporal load, as the decode kernels read keys and values.
__device__ __forceinline__ v4u ld(const uint4 *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
}

template <int NC, int SHAPE>
__global__ __launch_bounds__(1024) void probe_kernel(const uint4 *__restrict__ base,
                                                     const int32_t *__restrict__ chunk_ids,
                                                     int num_chunks, int chunks_per_group,
                                                     uint32_t *__restrict__ sink,
                                                     unsigned long long *__restrict__ times) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int first = blockIdx.x * chunks_per_group;
    const int last = min(first + chunks_per_group, num_chunks);
    uint32_t acc = 0;
    for (int k0 = first + w; k0 < last; k0 += nw * kInFlight) {
        v4u r[kInFlight][NC];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int k = k0 + u * nw;
            const int id = k < last ? (chunk_ids ? chunk_ids[k] : k) : (chunk_ids ? chunk_ids[first] : first);
            if (SHAPE == 0) {
                const uint4 *p = base + (size_t)id * (NC * 64) + lane;
#pragma unroll
                for (int c = 0; c < NC; ++c) r[u][c] = ld(p + c * 64);
            } else {
                const uint4 *p = base + (size_t)id * (NC * 64) + (lane & 15) * (NC * 4) + (lane >> 4);
#pragma unroll
                for (int c = 0; c < NC; ++c) r[u][c] = ld(p + c * 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
#pragma unroll
            for (int c = 0; c < NC; ++c) acc ^= r[u][c][0] ^ r[u][c][1] ^ r[u][c][2] ^ r[u][c][3];
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
    if (times != nullptr && threadIdx.x == 0) {
        // XCC_ID: hardware register 20, bits 0-3.
        const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u;
        times[3 * blockIdx.x + 0] = t0;
        times[3 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
        times[3 * blockIdx.x + 2] = xcc;
    }
}

}  // namespace

extern "C" int pa_probe_read(const void *base, const int32_t *chunk_ids, int num_chunks,
                             int chunk_bytes, int waves_per_group, int num_groups, int shape,
                             void *sink, void *stream) {
    if (!base || !sink || num_chunks <= 0 || num_groups <= 0) return 1;
    if (shape != 0 && !(shape == 1 && chunk_bytes == 4096)) return 1;
    if (waves_per_group < 1 || waves_per_group > 16) return 1;
    const int per = (num_chunks + num_groups - 1) / num_groups;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(num_groups), block(waves_per_group * 64);
    const uint4 *b = static_cast<const uint4 *>(base);
    uint32_t *o = static_cast<uint32_t *>(sink);
    if (shape == 1) {
        probe_kernel<4, 1><<<grid, block, 0, s>>>(b, chunk_ids, num_chunks, per, o, nullptr);
        return hipGetLastError() == hipSuccess ? 0 : 2;
    }
    switch (chunk_bytes) {
        case 1024: probe_kernel<1, 0><<<grid, block, 0, s>>>(b, chunk_ids, num_chunks, per, o, nullptr); break;
        case 4096: probe_kernel<4, 0><<<grid, block, 0, s>>>(b, chunk_ids, num_chunks, per, o, nullptr); break;
        case 16384: probe_kernel<16, 0><<<grid, block, 0, s>>>(b, chunk_ids, num_chunks, per, o, nullptr); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pa_probe_read_xcd(const void *base, const int32_t *chunk_ids, int num_chunks,
                                 int chunk_bytes, int waves_per_group, int num_groups, void *sink,
                                 void *times, void *stream) {
    if (!base || !sink || !times || num_chunks <= 0 || num_groups <= 0) return 1;
    if (waves_per_group < 1 || waves_per_group > 16 || chunk_bytes != 4096) return 1;
    const int per = (num_chunks + num_groups - 1) / num_groups;
    probe_kernel<4, 0><<<dim3(num_groups), dim3(waves_per_group * 64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4 *>(base), chunk_ids, num_chunks, per, static_cast<uint32_t *>(sink),
        static_cast<unsigned long long *>(times));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
