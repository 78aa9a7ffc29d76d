// pa_repack.hip -- gfx950 kernel that moves token-major paged caches into the
// split layout the attention kernels read (pure data movement, bit-exact).
//
// Method (project_6 commit pages): the pages gather a sequence's cache blocks
// by block id and permute each block into token order before the products
// (commit 15ef28e, "[OPT] Vectorize paged_attention_v2": the gather with
// .permute().reshape()); the order inside a block is the storage layout's
// choice.  A caller that stores K and V token-major -- [block][kv head][token]
// [d] -- hands them to this library once through this repack.
//
// Layouts, per (block, kv head) slab of 16 tokens x D elements of ES bytes,
// x = 16 / ES elements per 16-byte piece:
//   input keys and values   [token][d]
//   output keys             [d / x][token][x]  -- piece (c, t) = K[t][c x .. c x + x - 1],
//                                                 a contiguous 16 bytes of the input
//   output values           [d][token]         -- a transpose, staged through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kRepackThreads = 256;
constexpr int kRepackMaxDim = 512;

// One workgroup per slab, grid-stride over the slabs.  Either pair of pointers
// may be null (that cache is not repacked).
template <int ES>
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(const uint4 *__restrict__ kin,
                                                                const uint4 *__restrict__ vin,
                                                                uint4 *__restrict__ kout,
                                                                uint4 *__restrict__ vout,
                                                                long long slabs, int D) {
    constexpr int X = 16 / ES;
    __shared__ __attribute__((aligned(16))) char tile[kBlockTokens * kRepackMaxDim * ES];
    const int pieces = kBlockTokens * D / X;  // 16-byte pieces per slab
    const int per_row = D / X;                // pieces per token row of the input
    for (long long sl = blockIdx.x; sl < slabs; sl += gridDim.x) {
        const size_t base = (size_t)sl * pieces;
        if (kin != nullptr) {
            for (int p = threadIdx.x; p < pieces; p += kRepackThreads) {
                const int c = p / kBlockTokens, t = p - c * kBlockTokens;
                kout[base + p] = kin[base + (size_t)t * per_row + c];
            }
        }
        if (vin != nullptr) {
            for (int p = threadIdx.x; p < pieces; p += kRepackThreads)
                reinterpret_cast<uint4 *>(tile)[p] = vin[base + p];
            __syncthreads();
            // Output piece p: row d = p / (16 / X), tokens h X .. h X + X - 1 with
            // h = p % (16 / X); element (t, d) of the slab is at byte (t D + d) ES.
            constexpr int kHalves = kBlockTokens / X;
            for (int p = threadIdx.x; p < pieces; p += kRepackThreads) {
                const int d = p / kHalves, t0 = (p - d * kHalves) * X;
                uint32_t w[4];
                if constexpr (ES == 2) {
                    const uint16_t *e = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = (uint32_t)e[(t0 + 2 * i) * D + d] | ((uint32_t)e[(t0 + 2 * i + 1) * D + d] << 16);
                } else {
                    const uint32_t *e = reinterpret_cast<const uint32_t *>(tile);
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = e[(t0 + i) * D + d];
                }
                vout[base + p] = make_uint4(w[0], w[1], w[2], w[3]);
            }
            __syncthreads();  // the tile is refilled for the next slab
        }
    }
}

}  // namespace

int repack_max_dim() { return kRepackMaxDim; }

hipError_t launch_repack(const void *key_in, const void *value_in, void *key_out, void *value_out,
                         int num_blocks, int num_kv_heads, int head_dim, Dtype dtype,
                         hipStream_t stream) {
    const long long slabs = (long long)num_blocks * num_kv_heads;
    if (slabs <= 0) return hipSuccess;
    const int grid = (int)(slabs < 8192 ? slabs : 8192);
    auto *ki = static_cast<const uint4 *>(key_in);
    auto *vi = static_cast<const uint4 *>(value_in);
    auto *ko = static_cast<uint4 *>(key_out);
    auto *vo = static_cast<uint4 *>(value_out);
    if (dtype == Dtype::BF16)
        repack_kernel<2><<<grid, kRepackThreads, 0, stream>>>(ki, vi, ko, vo, slabs, head_dim);
    else
        repack_kernel<4><<<grid, kRepackThreads, 0, stream>>>(ki, vi, ko, vo, slabs, head_dim);
    return hipGetLastError();
}

}  // namespace pa
