// sbf_membench.hip -- matched ceilings for the filter kernels: the rate of
// uniformly random 32-byte shard reads (the query's and probe's access) and
// of random 32-byte shard OR-updates issued as the insert issues them (four
// adjacent lanes, one 64-bit atomic OR each), over a table of the filter's
// size; and the VALU issue rate of two instruction forms.  Measurement support for the roofline of "cuSBF: A
// Minimizer-Aware Bloom Filter for Genomic Sequence Data on Modern GPUs"
// §V-E (speed of light); none of it is part of the method.
//
// Every address is table + 4 * (h & (nshard - 1)) + q with q < 4, so every
// access stays inside the 4 * nshard words the caller passes.
#include <hip/hip_runtime.h>

#include "../../include/sbf.h"
#include "sbf_device.hpp"

namespace sbf {
namespace {

// Shard of operation j: the (j+1)-th SplitMix64 output of the seed.
__device__ __forceinline__ uint64_t op_hash(uint64_t seed, uint64_t j) { return splitmix_fin(seed + (j + 1u) * kGolden); }

// VALU issue rate: every lane runs `iters` rounds of eight independent
// instructions of one form, so no instruction waits on the one before it.
// kind 0: v_xor_b32 on VGPRs (the two-operand 32-bit logic, add and shift
// forms); kind 1: v_mad_u64_u32 (a 64-bit form).  Registers only; d_sink is
// written only if the XOR of the results hits a fixed value.
template <int KIND>
__global__ __launch_bounds__(256) void valu_rate_kernel(uint64_t iters, uint64_t* __restrict__ sink)
{
    uint32_t a0 = threadIdx.x, a1 = a0 + 1u, a2 = a0 + 2u, a3 = a0 + 3u, a4 = a0 + 4u, a5 = a0 + 5u, a6 = a0 + 6u,
             a7 = a0 + 7u;
    uint64_t d0 = a0, d1 = a1, d2 = a2, d3 = a3, d4 = a4, d5 = a5, d6 = a6, d7 = a7;
    const uint32_t b = 0x9E3779B9u ^ threadIdx.x;
    for (uint64_t i = 0; i < iters; ++i) {
        if constexpr (KIND == 0) {
            asm volatile(
                "v_xor_b32 %0, %0, %8\n v_xor_b32 %1, %1, %8\n v_xor_b32 %2, %2, %8\n v_xor_b32 %3, %3, %8\n"
                "v_xor_b32 %4, %4, %8\n v_xor_b32 %5, %5, %8\n v_xor_b32 %6, %6, %8\n v_xor_b32 %7, %7, %8"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(b));
        } else {
            asm volatile(
                "v_mad_u64_u32 %0, vcc, %8, %8, %0\n v_mad_u64_u32 %1, vcc, %8, %8, %1\n"
                "v_mad_u64_u32 %2, vcc, %8, %8, %2\n v_mad_u64_u32 %3, vcc, %8, %8, %3\n"
                "v_mad_u64_u32 %4, vcc, %8, %8, %4\n v_mad_u64_u32 %5, vcc, %8, %8, %5\n"
                "v_mad_u64_u32 %6, vcc, %8, %8, %6\n v_mad_u64_u32 %7, vcc, %8, %8, %7"
                : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3), "+v"(d4), "+v"(d5), "+v"(d6), "+v"(d7)
                : "v"(b)
                : "vcc");
        }
    }
    const uint64_t r = (uint64_t)(a0 ^ a1 ^ a2 ^ a3 ^ a4 ^ a5 ^ a6 ^ a7) ^ d0 ^ d1 ^ d2 ^ d3 ^ d4 ^ d5 ^ d6 ^ d7;
    if (r == 0x5EEDF00DCAFEBEEFull)
        sink[0] = r;
}

__global__ __launch_bounds__(256) void shard_reads_kernel(const uint64_t* __restrict__ table, uint64_t mask,
                                                          uint64_t n, uint64_t seed, uint64_t* __restrict__ sink)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t acc = 0;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        uint64_t w[4];
        load_shard(table, op_hash(seed, j) & mask, w);
        acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
    }
    // keeps the loads; the table never holds this value in practice, and a
    // store here would be harmless anyway
    if (acc == 0x5EEDF00DCAFEBEEFull)
        sink[0] = acc;
}

__global__ __launch_bounds__(256) void shard_ors_kernel(uint64_t* __restrict__ table, uint64_t mask, uint64_t n,
                                                        uint64_t seed)
{
    // four adjacent lanes per operation, lane q ORs word q
    const uint64_t stride = (uint64_t)gridDim.x * (blockDim.x / 4u);
    const uint32_t q = threadIdx.x & 3u;
    for (uint64_t j = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) / 4u; j < n; j += stride) {
        const uint64_t h = op_hash(seed, j);
        atomic_or_u64(table + 4u * (h & mask) + q, 1ull << ((h >> 58) ^ q));
    }
}

// Random 32-byte OR-updates in one of several forms (four adjacent lanes per
// operation, lane q updates word q): MODE 0 a 64-bit atomic OR at device
// scope, 1 the same at workgroup scope, 2 a plain load, OR and store (not
// atomic: concurrent updates of one word may be lost; a rate only).  PART
// confines the shards of workgroup b to the eighth of the table numbered
// b mod 8, the eighth its XCD would own under round-robin dispatch.
template <int MODE, bool PART>
__global__ __launch_bounds__(256) void shard_rmw_kernel(uint64_t* __restrict__ table, uint64_t mask, uint64_t n,
                                                        uint64_t seed)
{
    const uint64_t stride = (uint64_t)gridDim.x * (blockDim.x / 4u);
    const uint32_t q = threadIdx.x & 3u;
    const uint64_t part = (mask + 1u) / 8u;
    for (uint64_t j = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) / 4u; j < n; j += stride) {
        const uint64_t h = op_hash(seed, j);
        const uint64_t shard = PART ? (blockIdx.x % 8u) * part + (h & (part - 1u)) : (h & mask);
        uint64_t* p = table + 4u * shard + q;
        const uint64_t v = 1ull << ((h >> 58) ^ q);
        if constexpr (MODE == 0)
            __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else if constexpr (MODE == 1)
            __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
            *p = *p | v;
    }
}

uint32_t grid_for(uint64_t threads)
{
    uint64_t b = (threads + 255) / 256;
    if (b > 16384)
        b = 16384;
    return (uint32_t)(b ? b : 1);
}

bool pow2(uint64_t x) { return x && !(x & (x - 1)); }

// 8192 blocks of four waves: 32 waves per CU on 256 CUs, eight per SIMD.
constexpr uint32_t kValuBlocks = 8192;

}  // namespace
}  // namespace sbf

extern "C" {

int sbf_membench_shard_reads(const uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed, uint64_t* d_sink,
                             void* stream)
{
    if (!d_table || !d_sink || !sbf::pow2(nshard))
        return SBF_EINVAL;
    if (n == 0)
        return SBF_OK;
    (void)hipGetLastError();  // report this launch's error, not an earlier call's
    hipLaunchKernelGGL(sbf::shard_reads_kernel, dim3(sbf::grid_for(n)), dim3(256), 0, (hipStream_t)stream, d_table,
                       nshard - 1, n, seed, d_sink);
    return hipGetLastError() == hipSuccess ? SBF_OK : SBF_EDEVICE;
}

int sbf_membench_valu(uint32_t kind, uint64_t iters, uint64_t* d_sink, void* stream)
{
    if (!d_sink || kind > 1 || iters == 0 || iters > (1ull << 32))
        return SBF_EINVAL;
    (void)hipGetLastError();  // report this launch's error, not an earlier call's
    if (kind == 0)
        hipLaunchKernelGGL(sbf::valu_rate_kernel<0>, dim3(sbf::kValuBlocks), dim3(256), 0, (hipStream_t)stream, iters,
                           d_sink);
    else
        hipLaunchKernelGGL(sbf::valu_rate_kernel<1>, dim3(sbf::kValuBlocks), dim3(256), 0, (hipStream_t)stream, iters,
                           d_sink);
    return hipGetLastError() == hipSuccess ? SBF_OK : SBF_EDEVICE;
}

int sbf_membench_shard_ors(uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed, void* stream)
{
    if (!d_table || !sbf::pow2(nshard))
        return SBF_EINVAL;
    if (n == 0)
        return SBF_OK;
    (void)hipGetLastError();  // report this launch's error, not an earlier call's
    hipLaunchKernelGGL(sbf::shard_ors_kernel, dim3(sbf::grid_for(4 * n)), dim3(256), 0, (hipStream_t)stream, d_table,
                       nshard - 1, n, seed);
    return hipGetLastError() == hipSuccess ? SBF_OK : SBF_EDEVICE;
}

int sbf_membench_shard_rmw(uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed, uint32_t mode,
                           void* stream)
{
    const uint32_t form = mode & 3u;
    const bool part = (mode & 4u) != 0;
    if (!d_table || !sbf::pow2(nshard) || form > 2u || (mode & ~7u) || (part && nshard < 8))
        return SBF_EINVAL;
    if (n == 0)
        return SBF_OK;
    (void)hipGetLastError();  // report this launch's error, not an earlier call's
    const dim3 grid(sbf::grid_for(4 * n)), block(256);
    hipStream_t st = (hipStream_t)stream;
    const uint64_t mask = nshard - 1;
    switch (mode) {
    case 0: hipLaunchKernelGGL((sbf::shard_rmw_kernel<0, false>), grid, block, 0, st, d_table, mask, n, seed); break;
    case 1: hipLaunchKernelGGL((sbf::shard_rmw_kernel<1, false>), grid, block, 0, st, d_table, mask, n, seed); break;
    case 2: hipLaunchKernelGGL((sbf::shard_rmw_kernel<2, false>), grid, block, 0, st, d_table, mask, n, seed); break;
    case 4: hipLaunchKernelGGL((sbf::shard_rmw_kernel<0, true>), grid, block, 0, st, d_table, mask, n, seed); break;
    case 5: hipLaunchKernelGGL((sbf::shard_rmw_kernel<1, true>), grid, block, 0, st, d_table, mask, n, seed); break;
    default: hipLaunchKernelGGL((sbf::shard_rmw_kernel<2, true>), grid, block, 0, st, d_table, mask, n, seed); break;
    }
    return hipGetLastError() == hipSuccess ? SBF_OK : SBF_EDEVICE;
}

}  // extern "C"
