// sbf_membench.hip -- matched memory ceilings for the filter kernels: the
// rate of uniformly random 32-byte shard reads (the query's and probe's
// access) and of random 32-byte shard OR-updates issued as the insert issues
// them (four adjacent lanes, one 64-bit atomic OR each), over a table of the
// filter's size.  Measurement support for the roofline of "cuSBF: A
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

uint32_t grid_for(uint64_t threads)
{
    uint64_t b = (threads + 255) / 256;
    if (b > 16384)
        b = 16384;
    return (uint32_t)(b ? b : 1);
}

bool pow2(uint64_t x) { return x && !(x & (x - 1)); }

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

}  // extern "C"
