// q4_1 weight repack: canonical 20-byte blocks {fp16 d, fp16 m, u8 q[16]}
// into a code plane [rows, K/2] and a scale plane [rows, K/32] of {d, m}, so
// that a lane's 16 bytes of codes and 4 bytes of scales are each one aligned,
// coalesced load.  Same bytes, same count.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_prefill.h"

namespace moe {

__global__ void repack_q4_1_kernel(const uint8_t *canonical, uint8_t *packed, long long n_blocks_total,
                                   long long blocks_per_expert, int D, int F) {
    long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks_total) return;
    const long long e = b / blocks_per_expert, be = b % blocks_per_expert;
    // matrices: gate [F, D/32], up [F, D/32], down [D, F/32] blocks
    const long long g_blocks = (long long)F * (D / 32);
    long long m_off_blocks, bl;
    int rows, nb;
    if (be < g_blocks) {
        m_off_blocks = 0; bl = be; rows = F; nb = D / 32;
    } else if (be < 2 * g_blocks) {
        m_off_blocks = g_blocks; bl = be - g_blocks; rows = F; nb = D / 32;
    } else {
        m_off_blocks = 2 * g_blocks; bl = be - 2 * g_blocks; rows = D; nb = F / 32;
    }
    (void)nb;
    const uint8_t *src = canonical + (e * blocks_per_expert + be) * 20;
    const uint32_t *s32 = (const uint32_t *)src;  // 20-byte blocks are 4-byte aligned
    uint8_t *mat = packed + (e * blocks_per_expert + m_off_blocks) * 20;
    const long long mat_blocks = (long long)rows * nb;
    uint4 codes = make_uint4(s32[1], s32[2], s32[3], s32[4]);
    ((uint4 *)mat)[bl] = codes;
    ((uint32_t *)(mat + mat_blocks * 16))[bl] = s32[0];
}

hipError_t launch_repack_q4_1(const uint8_t *canonical, uint8_t *packed, int n_experts, int D, int F, hipStream_t st) {
    const long long bpe = 2LL * F * (D / 32) + (long long)D * (F / 32);
    const long long total = bpe * n_experts;
    const long long grid = (total + 255) / 256;
    hipLaunchKernelGGL(repack_q4_1_kernel, dim3((unsigned)grid), dim3(256), 0, st, canonical, packed, total, bpe, D, F);
    return hipGetLastError();
}

__global__ void repack_q4_1_matrix_kernel(const uint8_t *canonical, uint8_t *packed, long long n_blocks) {
    const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint32_t *s32 = (const uint32_t *)(canonical + b * 20);
    ((uint4 *)packed)[b] = make_uint4(s32[1], s32[2], s32[3], s32[4]);
    ((uint32_t *)(packed + n_blocks * 16))[b] = s32[0];
}

hipError_t launch_repack_q4_1_matrix(const uint8_t *canonical, uint8_t *packed, long long rows, int k,
                                     hipStream_t st) {
    const long long n_blocks = rows * (k / 32);
    const long long grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(repack_q4_1_matrix_kernel, dim3((unsigned)grid), dim3(256), 0, st, canonical, packed, n_blocks);
    return hipGetLastError();
}

}  // namespace moe
