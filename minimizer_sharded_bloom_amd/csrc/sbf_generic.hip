// sbf_generic.hip -- sequence packing, filter clearing, the per-k-mer kernels
// that serve any (k, m, s, H) with runtime loops, and the blocked Bloom
// filter comparator.
//
// Method: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on
// Modern GPUs" [cuSBF].  The generic kernels give one k-mer to each lane and
// recompute everything per k-mer, like the straightforward GPU scheme that
// [cuSBF] §I describes; the fast path for the configured parameter sets is in
// sbf_spec.hpp.
#include "sbf_device.hpp"
#include "sbf_internal.hpp"

namespace sbf {

// ---------------------------------------------------------------------------
// a1: ASCII -> 2-bit codes + validity ([cuSBF] §IV-A alphabet, §IV-F
// separators).  One lane per 16 bases: a 16-byte load, one code word and one
// 16-bit half of a validity word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void encode4(uint32_t four, uint32_t& code4, uint32_t& valid4)
{
    code4 = 0;
    valid4 = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t c = (four >> (8 * b)) & 0xFFu;
        // A=0x41 C=0x43 G=0x47 T=0x54 (and lower case): ((c>>1)^(c>>2))&3 = 0,1,2,3
        const uint32_t code = ((c >> 1) ^ (c >> 2)) & 3u;
        const uint32_t lc = c | 0x20u;
        const uint32_t ok = (lc == 'a') | (lc == 'c') | (lc == 'g') | (lc == 't');
        code4 |= code << (6 - 2 * b);
        valid4 |= ok << b;
    }
}

__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ ascii, uint64_t len,
                                                   uint32_t* __restrict__ codes, uint16_t* __restrict__ valid16,
                                                   uint64_t ncw, uint64_t nvh, int aligned16)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nvh)
        return;
    const uint64_t base = 16 * i;
    uint32_t q[4] = {0, 0, 0, 0};
    if (base + 16 <= len && aligned16) {
        const uint4 v = *reinterpret_cast<const uint4*>(ascii + base);
        q[0] = v.x;
        q[1] = v.y;
        q[2] = v.z;
        q[3] = v.w;
    } else if (base < len) {
        for (int j = 0; j < 16 && base + j < len; ++j)
            q[j >> 2] |= (uint32_t)(unsigned char)ascii[base + j] << (8 * (j & 3));
    }
    uint32_t code = 0, val = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t c4, v4;
        encode4(q[j], c4, v4);
        code |= c4 << (24 - 8 * j);
        val |= v4 << (4 * j);
    }
    if (base + 16 > len) {  // bases past len are invalid
        const uint32_t keep = base >= len ? 0u : (uint32_t)(len - base);
        val &= (1u << keep) - 1u;
    }
    if (i < ncw)
        codes[i] = code;
    valid16[i] = (uint16_t)val;
}

hipError_t launch_pack(const char* ascii, uint64_t len, uint32_t* codes, uint32_t* valid, hipStream_t st)
{
    if (len == 0)
        return hipSuccess;
    const uint64_t ncw = (len + 15) / 16;
    const uint64_t nvh = 2 * ((len + 31) / 32);  // 16-bit halves of validity words
    const int aligned = ((uintptr_t)ascii & 15u) == 0;
    const uint64_t blocks = (nvh + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, ascii, len, codes,
                       reinterpret_cast<uint16_t*>(valid), ncw, nvh, aligned);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint64_t* __restrict__ p, uint64_t n)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0;
}

hipError_t launch_fill_zero(uint64_t* p, uint64_t nwords, hipStream_t st)
{
    if (nwords == 0)
        return hipSuccess;
    uint64_t blocks = (nwords + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, p, nwords);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Generic per-k-mer kernels (runtime k, m, s, H; SBF and BBF).
// ---------------------------------------------------------------------------

// Packed value of the k-mer starting at base p (first base most significant).
__device__ __forceinline__ uint64_t kmer_at(const uint32_t* __restrict__ codes, uint64_t ncw, uint64_t p, uint32_t k)
{
    const uint64_t w = p >> 4;
    const uint32_t r = 2u * (uint32_t)(p & 15);
    const uint32_t d0 = ld_or0(codes, ncw, w), d1 = ld_or0(codes, ncw, w + 1), d2 = ld_or0(codes, ncw, w + 2);
    const uint64_t win = ((uint64_t)funnel_hi(d0, d1, r) << 32) | funnel_hi(d1, d2, r);
    return k >= 32 ? win : win >> (64 - 2 * k);
}

__device__ __forceinline__ bool kmer_valid_at(const uint32_t* __restrict__ valid, uint64_t nvw, uint64_t p, uint32_t k)
{
    const uint64_t w = p >> 5;
    const uint32_t off = (uint32_t)(p & 31);
    const uint64_t v01 = (uint64_t)ld_or0(valid, nvw, w) | ((uint64_t)ld_or0(valid, nvw, w + 1) << 32);
    const uint64_t win = off ? (v01 >> off) | ((uint64_t)ld_or0(valid, nvw, w + 2) << (64 - off)) : v01;
    const uint64_t need = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
    return (win & need) == need;
}

__device__ __forceinline__ uint64_t sub_rt(uint64_t x, uint32_t k, uint32_t j, uint32_t n)
{
    if (n >= 32)
        return x;
    return (x >> (2 * (k - n - j))) & ((1ull << (2 * n)) - 1ull);
}

// Shard and up to 4 sector masks of one k-mer ([cuSBF] Algorithm 1 for the
// SBF; one hash for the block and one for the bits for the BBF).
__device__ __forceinline__ uint32_t kmer_shard(uint64_t x, const Params& P, uint32_t shard_mask)
{
    if (P.kind == 1)
        return (uint32_t)hash_s(x) & shard_mask;
    uint64_t mn = ~0ull;
    for (uint32_t i = 0; i + P.m <= P.k; ++i) {
        const uint64_t h = hash_min(sub_rt(x, P.k, i, P.m));
        mn = h < mn ? h : mn;
    }
    return (uint32_t)mn & shard_mask;
}

__device__ __forceinline__ void kmer_masks(uint64_t x, const Params& P, uint64_t (&mk)[4])
{
    mk[0] = mk[1] = mk[2] = mk[3] = 0;
    if (P.kind == 1) {
        const uint64_t hb = hash_s(hash_s(x));
        for (uint32_t t = 0; t < P.H; ++t)
            mk[t & 3] |= 1ull << bit_addr_rt(hb, t, P.H);
        return;
    }
    for (uint32_t j = 0; j + P.s <= P.k; ++j) {
        const uint64_t h = hash_s(sub_rt(x, P.k, j, P.s));
        for (uint32_t t = 0; t < P.H; ++t)
            mk[t & 3] |= 1ull << bit_addr_rt(h, t, P.H);
    }
}

__global__ __launch_bounds__(256) void generic_insert_kernel(SeqArgs a, Params P)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < a.nk; p += stride) {
        if (!kmer_valid_at(a.valid, a.nvw, p, P.k))
            continue;
        const uint64_t x = kmer_at(a.codes, a.ncw, p, P.k);
        const uint32_t sh = kmer_shard(x, P, a.shard_mask);
        uint64_t mk[4];
        kmer_masks(x, P, mk);
        uint64_t* base = a.filter + 4ull * sh;
        for (int q = 0; q < 4; ++q)
            if (mk[q])
                atomic_or_u64(base + q, mk[q]);
    }
}

// Every query mask bit must be set in the shard.
__device__ __forceinline__ bool shard_has(const uint64_t* __restrict__ filter, uint32_t sh, const uint64_t (&mk)[4])
{
    uint64_t w[4];
    load_shard(filter, sh, w);
    return ((w[0] & mk[0]) == mk[0]) & ((w[1] & mk[1]) == mk[1]) & ((w[2] & mk[2]) == mk[2]) &
           ((w[3] & mk[3]) == mk[3]);
}

// One k-mer per lane; grid-stride over 64-aligned groups so each wave's
// ballot is one output word.
__global__ __launch_bounds__(256) void generic_query_kernel(SeqArgs a, Params P)
{
    const uint64_t nk_pad = (a.nk + 63) & ~63ull;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t p0 = (uint64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63u); p0 < nk_pad; p0 += stride) {
        const uint64_t p = p0 + (threadIdx.x & 63u);
        bool pres = false;
        if (p < a.nk && kmer_valid_at(a.valid, a.nvw, p, P.k)) {
            const uint64_t x = kmer_at(a.codes, a.ncw, p, P.k);
            uint64_t mk[4];
            kmer_masks(x, P, mk);
            pres = shard_has(a.filter, kmer_shard(x, P, a.shard_mask), mk);
        }
        const uint64_t word = __ballot(pres);
        if ((threadIdx.x & 63u) == 0)
            a.out[p0 >> 6] = word;
    }
}

__global__ __launch_bounds__(256) void generic_probe_kernel(ProbeArgs a, Params P)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t cnt = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += stride) {
        const uint64_t x = splitmix_fin(a.seed + (i + 1) * kGolden) >> (64 - 2 * P.k);
        uint64_t mk[4];
        kmer_masks(x, P, mk);
        cnt += shard_has(a.filter, kmer_shard(x, P, a.shard_mask), mk);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

static uint32_t grid_for(uint64_t n)
{
    uint64_t b = (n + 255) / 256;
    if (b > 65536)
        b = 65536;
    return (uint32_t)(b ? b : 1);
}

static hipError_t gen_insert(const SeqArgs& a, const Params& P)
{
    hipLaunchKernelGGL(generic_insert_kernel, dim3(grid_for(a.nk)), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

static hipError_t gen_query(const SeqArgs& a, const Params& P)
{
    hipLaunchKernelGGL(generic_query_kernel, dim3(grid_for((a.nk + 63) & ~63ull)), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

static hipError_t gen_probe(const ProbeArgs& a, const Params& P)
{
    if (a.n == 0)
        return hipSuccess;
    uint64_t b = (a.n + 255) / 256;
    if (b > 8192)
        b = 8192;
    hipLaunchKernelGGL(generic_probe_kernel, dim3((uint32_t)b), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

KernelSet generic_kernels()
{
    KernelSet ks;
    ks.insert = &gen_insert;
    ks.query = &gen_query;
    ks.probe = &gen_probe;
    ks.specialized = 0;
    return ks;
}

}  // namespace sbf
