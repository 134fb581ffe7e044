// sbf_wide.hpp -- compile-time specialized gfx950 kernels of the wide-block
// variant: 512-bit blocks, each hash index addressing any bit of the block
// (the layout "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence
// Data on Modern GPUs" §V-D attributes to the CPU Super Bloom reference).
//
// The front end -- lanes, packed bases, minimizer keys, run starts, the wave
// scan and per-k-mer records -- is that of sbf_spec.hpp.  What differs is the
// bit work: a hash may land in any of the block's 8 words, so instead of
// per-sector register masks the kernels keep each segment's block in LDS and
// address its 32-bit words directly.
//  - Every s-mer is hashed once (own positions, halo from lane+1 by DPP); its
//    H bit addresses a and LDS byte offsets 4 * (a / 32) are kept for the Z
//    k-mers that contain it.
//  - Query: k-mer i reads, for each of its Z*H addresses, the 32-bit word of
//    its record and tests bit a mod 32.
//  - Insert: k-mer i ORs the bits of its newest s-mer into its record with an
//    LDS atomic, and a run's first k-mer also ORs those of the Z-1 s-mers
//    before; a run cut by a lane boundary shares one record, the atomics make
//    that free.  Then 8 adjacent lanes OR one record's 8 words into the
//    filter, one 64-byte request per run.
//  - Probe: each lane stages its random k-mer's block in a private LDS slot
//    and tests it the same way.
#pragma once

#include "sbf_spec.hpp"

namespace sbf {

// LDS records per wave: 12 per lane's worth of k-mers (192 for 16 k-mers per
// lane, 384 for 32); a workgroup holds 4 waves, or 2 when a lane has 32
// k-mers, so either way it takes about 52 KB of LDS and a CU holds three.
template <class C>
struct WideShape {
    static constexpr int kSlots = 12 * C::KL;
    static constexpr int kWavesPerBlock = C::KL == 32 ? 2 : 4;
};

template <class C>
struct WideLds {
    static constexpr int NW = WideShape<C>::kWavesPerBlock, NS = WideShape<C>::kSlots;
    uint32_t idx[NW][NS + 1];
    alignas(16) uint32_t words[NW][NS + 1][16];  // 512-bit blocks as 16 32-bit words
};

// Streaming s-mer bit addresses: positions 0 .. KL+Z-2 of the lane (own KL,
// halo Z-1 from lane l+1); for each, H addresses and LDS byte offsets.
template <class C>
struct WideAddr {
    static constexpr int Z = C::Z, H = C::H, NH = Z > 1 ? Z - 1 : 1;
    uint32_t a[C::NZ][H];    // 9-bit addresses
    uint32_t off[C::NZ][H];  // 4 * (a / 32): byte offset of the word in the block
    uint64_t head[NH], halo[NH];

    __device__ __forceinline__ void init(const uint32_t (&D)[C::ND])
    {
        static_for<0, Z - 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            head[q] = smer_hash_at<C, q>(D);
        });
        static_for<0, Z - 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            halo[q] = from_next_lane(head[q]);
        });
    }

    template <int Q>
    __device__ __forceinline__ uint64_t hash_of(const uint32_t (&D)[C::ND])
    {
        if constexpr (Q < Z - 1)
            return head[Q];
        else if constexpr (Q < C::KL)
            return smer_hash_at<C, Q>(D);
        else
            return halo[Q - C::KL];
    }

    template <int Q>
    __device__ __forceinline__ void compute(const uint32_t (&D)[C::ND])
    {
        const uint64_t h = hash_of<Q>(D);
#pragma unroll
        for (int t = 0; t < H; ++t) {
            a[Q][t] = bit_addr_wide<H>(h, t);
            off[Q][t] = (a[Q][t] >> 3) & 0x3Cu;
        }
    }

    // Addresses of the s-mers first needed by k-mer I: 0..Z-1 at I = 0, then I+Z-1.
    template <int I>
    __device__ __forceinline__ void step(const uint32_t (&D)[C::ND])
    {
        constexpr int qn = I == 0 ? 0 : I + Z - 1;
        static_for<qn, I + Z>([&](auto qc) { compute<decltype(qc)::value>(D); });
    }
};

// All Z*H bits of k-mer I set in the LDS block at `blk`?
template <class C, int I>
__device__ __forceinline__ uint32_t wide_test(const WideAddr<C>& wa, const char* blk)
{
    uint32_t acc = ~0u;
#pragma unroll
    for (int j = 0; j < C::Z; ++j) {
#pragma unroll
        for (int t = 0; t < C::H; ++t) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + wa.off[I + j][t]);
            acc &= w >> (wa.a[I + j][t] & 31u);
        }
    }
    return acc & 1u;
}

// ---------------------------------------------------------------------------
// Query
// ---------------------------------------------------------------------------

// Per-k-mer path for waves whose segments exceed the LDS records: each k-mer
// on its own, its block's words read from the filter.
template <class C>
__device__ __forceinline__ uint32_t wide_query_lane_direct(const SeqArgs& a, const uint32_t (&D)[C::ND], uint32_t vk)
{
    uint32_t bits = 0;
    for (int i = 0; i < C::KL; ++i) {
        if (!((vk >> i) & 1u))
            continue;
        const bool hi16 = i >= 16;
        const uint32_t d0 = hi16 ? D[1] : D[0];
        const uint32_t d1 = hi16 ? D[2] : D[1];
        const uint32_t d2 = hi16 ? D[C::ND - 1] : D[2];
        const uint32_t r = 2u * (uint32_t)(i & 15);
        const uint64_t win = ((uint64_t)funnel_hi(d0, d1, r) << 32) | funnel_hi(d1, d2, r);
        const uint64_t x = top_bases(win, C::k);
        uint64_t mn = ~0ull;
#pragma unroll
        for (int j = 0; j < C::W; ++j) {
            const uint64_t h = hash_min(sub_bases<C::k, C::m>(x, j));
            mn = h < mn ? h : mn;
        }
        const uint32_t* blk = reinterpret_cast<const uint32_t*>(a.filter + 8ull * ((uint32_t)mn & a.shard_mask));
        uint32_t acc = ~0u;
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            const uint64_t h = hash_s(sub_bases<C::k, C::s>(x, j));
#pragma unroll
            for (int t = 0; t < C::H; ++t) {
                const uint32_t ad = bit_addr_wide<C::H>(h, t);
                acc &= blk[ad >> 5] >> (ad & 31u);
            }
        }
        bits |= (acc & 1u) << i;
    }
    return bits;
}

template <class C>
__global__ __launch_bounds__(256) void wide_query_kernel(SeqArgs a)
{
    __shared__ WideLds<C> lds;
    constexpr uint32_t kSlotsW = WideShape<C>::kSlots;
    const uint64_t nk_pad = round64(a.nk);
    const LaneCtx<C> c = lane_ctx<C>(nk_pad);
    if (!c.live)
        return;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t D[C::ND];
    load_codes<C>(a, c, D);
    const uint32_t vk = lane_valid<C>(a, c);
    uint32_t total;
    uint32_t rec[C::KL];
    {
        uint32_t shard[C::KL];
        lane_shards<C>(D, shard);
        uint32_t gs, first;
        total = query_records<C>(vk, shard, c.lane, rec, gs, first);
        if (total <= (uint32_t)kSlotsW) {
#pragma unroll
            for (int i = 0; i < C::KL; ++i)
                lds.idx[wv][rec[i]] = shard[i];
            point_gaps_at_shard0<C>(lds.idx[wv], vk, gs, first);
        }
    }
    uint32_t bits;
    if (total <= (uint32_t)kSlotsW) {
        wave_lds_sync();
        gather_records<64, kSlotsW>(a.filter, a.shard_mask, lds.idx[wv],
                                    reinterpret_cast<char*>(&lds.words[wv][0][0]), total, c.lane);
        wave_lds_sync();

        WideAddr<C> wa;
        wa.init(D);
        const char* base = reinterpret_cast<const char*>(&lds.words[wv][0][0]);
        bits = 0;
        static_for<0, C::KL>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            wa.template step<i>(D);
            const uint32_t hit = wide_test<C, i>(wa, base + 64u * rec[i]);
            bits = shift_in(bits, __builtin_amdgcn_ballot_w64(hit != 0));  // k-mer i lands at bit KL-1-i
            step_fence(D);
        });
        bits = (__builtin_bitreverse32(bits) >> (32 - C::KL)) & vk;
    } else {
        bits = wide_query_lane_direct<C>(a, D, vk);
    }
    if (c.lane < (uint32_t)C::LW && c.p0 < nk_pad) {
        if constexpr (C::KL == 16)
            reinterpret_cast<uint16_t*>(a.out)[c.p0 >> 4] = (uint16_t)bits;
        else
            reinterpret_cast<uint32_t*>(a.out)[c.p0 >> 5] = bits;
    }
}

// ---------------------------------------------------------------------------
// Insert
// ---------------------------------------------------------------------------

// Per-k-mer path for waves whose runs exceed the LDS records: every bit of
// every valid k-mer straight to the filter.
template <class C>
__device__ __forceinline__ void wide_insert_lane_direct(const SeqArgs& a, const uint32_t (&D)[C::ND], uint32_t vk)
{
    for (int i = 0; i < C::KL; ++i) {
        if (!((vk >> i) & 1u))
            continue;
        const bool hi16 = i >= 16;
        const uint32_t d0 = hi16 ? D[1] : D[0];
        const uint32_t d1 = hi16 ? D[2] : D[1];
        const uint32_t d2 = hi16 ? D[C::ND - 1] : D[2];
        const uint32_t r = 2u * (uint32_t)(i & 15);
        const uint64_t win = ((uint64_t)funnel_hi(d0, d1, r) << 32) | funnel_hi(d1, d2, r);
        const uint64_t x = top_bases(win, C::k);
        uint64_t mn = ~0ull;
#pragma unroll
        for (int j = 0; j < C::W; ++j) {
            const uint64_t h = hash_min(sub_bases<C::k, C::m>(x, j));
            mn = h < mn ? h : mn;
        }
        uint64_t* blk = a.filter + 8ull * ((uint32_t)mn & a.shard_mask);
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            const uint64_t h = hash_s(sub_bases<C::k, C::s>(x, j));
#pragma unroll
            for (int t = 0; t < C::H; ++t) {
                const uint32_t ad = bit_addr_wide<C::H>(h, t);
                atomic_or_u64(blk + (ad >> 6), 1ull << (ad & 63u));
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(256) void wide_insert_kernel(SeqArgs a)
{
    __shared__ WideLds<C> lds;
    constexpr uint32_t kSlotsW = WideShape<C>::kSlots;
    const LaneCtx<C> c = lane_ctx<C>(a.nk);
    if (!c.live)
        return;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t D[C::ND];
    load_codes<C>(a, c, D);
    const uint32_t vk = lane_valid<C>(a, c);
    uint32_t total, st;
    uint32_t rec[C::KL];
    {
        uint32_t shard[C::KL];
        lane_shards<C>(D, shard);
        st = run_starts<C>(vk, shard);
        const uint32_t cin = continues_previous<C>(vk, shard, c.lane) ? 1u : 0u;
        const uint32_t nseg = __popc(st) - cin;
        const uint32_t incl = wave_incl_scan(nseg);
        total = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t first = incl - nseg - cin;
#pragma unroll
        for (int i = 0; i < C::KL; ++i)
            rec[i] = (__popc(st & ((2u << i) - 1u)) + first) * ((vk >> i) & 1u);
        if (total <= (uint32_t)kSlotsW) {
#pragma unroll
            for (int i = 0; i < C::KL; ++i)
                lds.idx[wv][rec[i]] = shard[i];
        }
    }
    if (total > (uint32_t)kSlotsW) {
        wide_insert_lane_direct<C>(a, D, vk);
        return;
    }
    // zero the records 0 .. total, 16 bytes per lane per round
    for (uint32_t r = c.lane; r < 4u * (total + 1u); r += 64u)
        reinterpret_cast<ulonglong2*>(lds.words[wv][r >> 2])[r & 3u] = ulonglong2{0, 0};
    wave_lds_sync();

    WideAddr<C> wa;
    wa.init(D);
    char* base = reinterpret_cast<char*>(&lds.words[wv][0][0]);
    static_for<0, C::KL>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        wa.template step<i>(D);
        char* blk = base + 64u * rec[i];  // invalid k-mers: record 0, never flushed
        // the newest s-mer of k-mer i
#pragma unroll
        for (int t = 0; t < C::H; ++t)
            __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(blk + wa.off[i + C::Z - 1][t]),
                                  1u << (wa.a[i + C::Z - 1][t] & 31u), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WAVEFRONT);
        // a run's first k-mer: the s-mers before its newest
        if ((st >> i) & 1u) {
#pragma unroll
            for (int j = 0; j < C::Z - 1; ++j)
#pragma unroll
                for (int t = 0; t < C::H; ++t)
                    __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(blk + wa.off[i + j][t]),
                                          1u << (wa.a[i + j][t] & 31u), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
        step_fence(D);
    });
    wave_lds_sync();

    // flush: lane -> (record 1 + lane/8 + 8 j, word lane & 7)
    const uint32_t q = c.lane & 7u;
    for (uint32_t r = 1u + (c.lane >> 3); r <= total; r += 8u) {
        const uint64_t m = reinterpret_cast<const uint64_t*>(lds.words[wv][r])[q];
        if (m)
            atomic_or_u64(a.filter + 8ull * (lds.idx[wv][r] & a.shard_mask) + q, m);
    }
}

// ---------------------------------------------------------------------------
// Probe ([cuSBF] §V-D): random k-mers, each block staged in the lane's LDS slot
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) void wide_probe_kernel(ProbeArgs a)
{
    __shared__ uint32_t slot[256][16];
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t* mine = slot[threadIdx.x];
    uint32_t cnt = 0;
    for (uint64_t i = tid; i < a.n; i += stride) {
        const uint64_t x = splitmix_fin(a.seed + (i + 1) * kGolden) >> (64 - 2 * C::k);
        uint64_t mn = ~0ull;
#pragma unroll
        for (int j = 0; j < C::W; ++j) {
            const uint64_t h = hash_min(sub_bases<C::k, C::m>(x, j));
            mn = h < mn ? h : mn;
        }
        const ulonglong2* blk = reinterpret_cast<const ulonglong2*>(a.filter + 8ull * ((uint32_t)mn & a.shard_mask));
        const ulonglong2 b0 = blk[0], b1 = blk[1], b2 = blk[2], b3 = blk[3];
        ulonglong2* m2 = reinterpret_cast<ulonglong2*>(mine);
        m2[0] = b0;
        m2[1] = b1;
        m2[2] = b2;
        m2[3] = b3;
        uint32_t acc = ~0u;
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            const uint64_t h = hash_s(sub_bases<C::k, C::s>(x, j));
#pragma unroll
            for (int t = 0; t < C::H; ++t) {
                const uint32_t ad = bit_addr_wide<C::H>(h, t);
                acc &= mine[ad >> 5] >> (ad & 31u);
            }
        }
        cnt += acc & 1u;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

template <class C>
hipError_t launch_wide_insert(const SeqArgs& a, const Params&)
{
    constexpr uint64_t nw = WideShape<C>::kWavesPerBlock;
    const uint64_t waves = (a.nk + C::KPW - 1) / C::KPW;
    const uint64_t blocks = (waves + nw - 1) / nw;
    hipLaunchKernelGGL(wide_insert_kernel<C>, dim3((uint32_t)blocks), dim3(64 * nw), 0, a.stream, a);
    return hipGetLastError();
}

template <class C>
hipError_t launch_wide_query(const SeqArgs& a, const Params&)
{
    constexpr uint64_t nw = WideShape<C>::kWavesPerBlock;
    const uint64_t waves = (round64(a.nk) + C::KPW - 1) / C::KPW;
    const uint64_t blocks = (waves + nw - 1) / nw;
    hipLaunchKernelGGL(wide_query_kernel<C>, dim3((uint32_t)blocks), dim3(64 * nw), 0, a.stream, a);
    return hipGetLastError();
}

template <class C>
hipError_t launch_wide_probe(const ProbeArgs& a, const Params&)
{
    uint64_t blocks = (a.n + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(wide_probe_kernel<C>, dim3((uint32_t)blocks), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

template <int K, int M, int S, int H>
KernelSet wide_set()
{
    using C = Cfg<K, M, S, H>;
    KernelSet ks;
    ks.insert = &launch_wide_insert<C>;
    ks.query = &launch_wide_query<C>;
    ks.probe = &launch_wide_probe<C>;
    ks.specialized = 1;
    return ks;
}

}  // namespace sbf
