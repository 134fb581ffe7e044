// sbf_spec.hpp -- compile-time specialized gfx950 kernels of the Super Bloom
// filter ([cuSBF] §IV-C..E, §IV-G "compile-time specialization").
//
// Work layout (one wave64 = 64 lanes, no LDS, no barriers):
//  - A wave owns KPW = 63 * KL consecutive k-mer starts.  Lane l < 63 owns
//    the KL consecutive k-mers starting at p0 = wave_start + KL * l; lane 63
//    only computes hashes for the halo of lane 62.
//  - Every lane loads its packed bases (KL/16 + 2 words, coalesced across the
//    wave), then computes the m-mer hash and the s-mer hash of its own KL
//    positions exactly once; the (w-1) m-mer hashes and (k-s) s-mer hashes past
//    its range come from lane l+1 through a lane shift.  No hash is computed
//    twice (apart from lane 63's 1/64 share).
//  - The minimizer of each k-mer is a sliding-window minimum over the w m-mer
//    hashes (van Herk / Gil-Werman block prefix and suffix minima, block = w).
//  - Insert: consecutive valid k-mers of a lane with the same shard form a
//    run ([cuSBF] §IV-D, Fig. 3); the run ORs its s-mer bits into four 64-bit
//    sector masks in registers and issues one atomic OR per used sector when
//    it ends.  Query: a lane loads a shard once per run and tests every k-mer
//    of the run against the registers ([cuSBF] §IV-E shard sharing); the KL
//    answer bits of a lane are one 16/32-bit store.
#pragma once

#include "sbf_device.hpp"
#include "sbf_internal.hpp"

namespace sbf {

template <int K_, int M_, int S_, int H_>
struct Cfg {
    static constexpr int k = K_, m = M_, s = S_, H = H_;
    static constexpr int W = k - m + 1;    // m-mers per k-mer
    static constexpr int Z = k - s + 1;    // s-mers per k-mer (Findere z+1)
    static constexpr int HALO = (W - 1 > Z - 1) ? W - 1 : Z - 1;
    static constexpr int KL = HALO <= 16 ? 16 : 32;  // k-mers per lane
    static constexpr int LW = 63;                    // working lanes per wave
    static constexpr int KPW = KL * LW;              // k-mers per wave
    static constexpr int ND = KL / 16 + 2;           // code words per lane
    static constexpr int NS = H < 4 ? H : 4;         // sectors in use
    static constexpr int NM = KL + W - 1;            // m-mer hashes per lane
    static constexpr int NZ = KL + Z - 1;            // s-mer hashes per lane
    static_assert(1 <= m && m <= k && k <= 32 && 1 <= s && s <= k && H >= 1, "bad parameters");
};

// Window of N bases starting at base j of a packed KK-mer x.
template <int KK, int N>
__device__ __forceinline__ uint64_t sub_bases(uint64_t x, int j)
{
    if constexpr (N >= 32)
        return x;
    else
        return (x >> (2 * (KK - N - j))) & ((1ull << (2 * N)) - 1ull);
}

// Answer words are written in KL-bit pieces; the grid covers nk rounded up
// to 64 so every piece of every output word is written.
__host__ __device__ inline uint64_t round64(uint64_t x) { return (x + 63) & ~63ull; }

template <class C>
struct LaneCtx {
    uint64_t p0;        // first k-mer of this lane
    uint32_t lane;
    bool live;          // wave has work
};

template <class C>
__device__ __forceinline__ LaneCtx<C> lane_ctx(uint64_t nk_pad)
{
    LaneCtx<C> c;
    c.lane = threadIdx.x & 63u;
    const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint64_t wstart = wave * (uint64_t)C::KPW;
    c.live = wstart < nk_pad;
    c.p0 = wstart + (uint64_t)C::KL * c.lane;
    return c;
}

template <class C>
__device__ __forceinline__ void load_codes(const SeqArgs& a, uint64_t p0, uint32_t (&D)[C::ND])
{
    const uint64_t w0 = p0 >> 4;
#pragma unroll
    for (int j = 0; j < C::ND; ++j)
        D[j] = ld_or0(a.codes, a.ncw, w0 + j);
}

// Shards of the lane's KL k-mers: one m-mer hash per own position, halo from
// lane+1, then van Herk sliding minimum with block size W.
template <class C>
__device__ __forceinline__ void lane_shards(const uint32_t (&D)[C::ND], uint32_t shard_mask, uint32_t (&shard)[C::KL])
{
    constexpr int W = C::W, KL = C::KL, NM = C::NM;
    uint64_t hm[NM];
#pragma unroll
    for (int i = 0; i < KL; ++i)
        hm[i] = hash_min(top_bases(stream_window<C::ND>(D, i), C::m));
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        hm[KL + j] = __shfl_down(hm[j], 1);
    if constexpr (W == 1) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
            shard[i] = (uint32_t)hm[i] & shard_mask;
    } else {
        // suffix minima inside blocks [bW, bW+W) clipped to NM, prefix minima likewise
        uint64_t suf[NM], pre[NM];
#pragma unroll
        for (int j = NM - 1; j >= 0; --j) {
            const bool block_end = ((j % W) == W - 1) || (j == NM - 1);
            suf[j] = block_end ? hm[j] : (hm[j] < suf[j + 1 < NM ? j + 1 : j] ? hm[j] : suf[j + 1 < NM ? j + 1 : j]);
        }
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            const bool block_start = (j % W) == 0;
            pre[j] = block_start ? hm[j] : (hm[j] < pre[j > 0 ? j - 1 : 0] ? hm[j] : pre[j > 0 ? j - 1 : 0]);
        }
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            uint64_t mn;
            if (i % W == 0) {
                mn = suf[i];
            } else {
                const uint64_t a = suf[i], b = pre[i + W - 1];
                mn = a < b ? a : b;
            }
            shard[i] = (uint32_t)mn & shard_mask;
        }
    }
}

// s-mer hashes of positions 0 .. KL+Z-2 (own KL, halo from lane+1).
template <class C>
__device__ __forceinline__ void lane_smer_hashes(const uint32_t (&D)[C::ND], uint64_t (&hs)[C::NZ])
{
#pragma unroll
    for (int i = 0; i < C::KL; ++i)
        hs[i] = hash_s(top_bases(stream_window<C::ND>(D, i), C::s));
#pragma unroll
    for (int j = 0; j < C::Z - 1; ++j)
        hs[C::KL + j] = __shfl_down(hs[j], 1);
}

// Valid-k-mer bits of the lane (bit i: k-mer p0+i is valid and < nk).
template <class C>
__device__ __forceinline__ uint32_t lane_valid(const SeqArgs& a, uint64_t p0, uint32_t lane)
{
    if (lane >= (uint32_t)C::LW || p0 >= a.nk)
        return 0u;
    uint64_t v = run_and<C::k>(valid_window64(a.valid, a.nvw, p0));
    const uint64_t rem = a.nk - p0;
    if (rem < (uint64_t)C::KL)
        v &= (1ull << rem) - 1ull;
    return (uint32_t)v & (uint32_t)((C::KL == 32) ? 0xFFFFFFFFu : ((1u << C::KL) - 1u));
}

// Sector masks of one s-mer hash: hash index t sets one bit in word t mod 4.
template <class C>
__device__ __forceinline__ void smer_masks(uint64_t h, uint64_t (&mk)[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        mk[q] = 0;
#pragma unroll
    for (int t = 0; t < C::H; ++t)
        mk[t & 3] |= 1ull << bit_addr<C::H>(h, t);
}

template <class C>
__device__ __forceinline__ void flush_run(uint64_t* __restrict__ filter, uint32_t shard, const uint64_t (&Wm)[4])
{
    uint64_t* base = filter + 4ull * shard;
#pragma unroll
    for (int q = 0; q < C::NS; ++q)
        atomic_or_u64(base + q, Wm[q]);
}

template <class C>
__global__ __launch_bounds__(256) void sbf_insert_kernel(SeqArgs a)
{
    const LaneCtx<C> c = lane_ctx<C>(a.nk);
    if (!c.live)
        return;  // whole wave
    uint32_t D[C::ND];
    load_codes<C>(a, c.p0, D);
    uint32_t shard[C::KL];
    lane_shards<C>(D, a.shard_mask, shard);
    uint64_t hs[C::NZ];
    lane_smer_hashes<C>(D, hs);
    const uint32_t vk = lane_valid<C>(a, c.p0, c.lane);
    if (vk == 0)
        return;

    uint64_t Wm[4] = {0, 0, 0, 0};
    bool open = false;
    uint32_t cur = 0;
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
        const bool vi = (vk >> i) & 1u;
        const bool cont = open && vi && shard[i] == cur;
        if (open && !cont)
            flush_run<C>(a.filter, cur, Wm);
        if (vi) {
            if (!cont) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    Wm[q] = 0;
#pragma unroll
                for (int j = 0; j < C::Z - 1; ++j) {
                    uint64_t mk[4];
                    smer_masks<C>(hs[i + j], mk);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        Wm[q] |= mk[q];
                }
            }
            uint64_t mk[4];
            smer_masks<C>(hs[i + C::Z - 1], mk);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Wm[q] |= mk[q];
            cur = shard[i];
        }
        open = vi;
    }
    if (open)
        flush_run<C>(a.filter, cur, Wm);
}

template <class C>
__device__ __forceinline__ bool smer_hits(const uint64_t (&w)[4], uint64_t h)
{
    uint64_t acc = ~0ull;
#pragma unroll
    for (int t = 0; t < C::H; ++t)
        acc &= w[t & 3] >> bit_addr<C::H>(h, t);
    return acc & 1ull;
}

template <class C>
__global__ __launch_bounds__(256) void sbf_query_kernel(SeqArgs a)
{
    const uint64_t nk_pad = round64(a.nk);
    const LaneCtx<C> c = lane_ctx<C>(nk_pad);
    if (!c.live)
        return;
    uint32_t D[C::ND];
    load_codes<C>(a, c.p0, D);
    uint32_t shard[C::KL];
    lane_shards<C>(D, a.shard_mask, shard);
    uint64_t hs[C::NZ];
    lane_smer_hashes<C>(D, hs);
    const uint32_t vk = lane_valid<C>(a, c.p0, c.lane);

    uint32_t bits = 0;
    uint64_t w[4] = {0, 0, 0, 0};
    bool have = false;
    uint32_t cur = 0;
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
        const bool vi = (vk >> i) & 1u;
        if (vi && (!have || shard[i] != cur)) {
            load_shard(a.filter, shard[i], w);
            cur = shard[i];
            have = true;
        }
        bool pres = vi;
#pragma unroll
        for (int j = 0; j < C::Z; ++j)
            pres &= smer_hits<C>(w, hs[i + j]);
        bits |= (uint32_t)pres << i;
    }
    if (c.lane < (uint32_t)C::LW && c.p0 < nk_pad) {
        if constexpr (C::KL == 16)
            reinterpret_cast<uint16_t*>(a.out)[c.p0 >> 4] = (uint16_t)bits;
        else
            reinterpret_cast<uint32_t*>(a.out)[c.p0 >> 5] = bits;
    }
}

// [cuSBF] §V-D: n uniformly random k-mers from the SplitMix64 stream, each
// queried on its own (minimizer over its w m-mers, one shard load, all s-mers).
template <class C>
__global__ __launch_bounds__(256) void sbf_probe_kernel(ProbeArgs a)
{
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t cnt = 0;
    for (uint64_t i = tid; i < a.n; i += stride) {
        const uint64_t x = splitmix_fin(a.seed + (i + 1) * kGolden) >> (64 - 2 * C::k);
        uint64_t mn = ~0ull;
#pragma unroll
        for (int j = 0; j < C::W; ++j) {
            const uint64_t h = hash_min(sub_bases<C::k, C::m>(x, j));
            mn = h < mn ? h : mn;
        }
        uint64_t w[4];
        load_shard(a.filter, (uint32_t)mn & a.shard_mask, w);
        bool pres = true;
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            pres &= smer_hits<C>(w, hash_s(sub_bases<C::k, C::s>(x, j)));
        }
        cnt += pres;
    }
    // wave reduction, one atomic per wave
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

template <class C>
hipError_t launch_insert(const SeqArgs& a, const Params&)
{
    const uint64_t waves = (a.nk + C::KPW - 1) / C::KPW;
    const uint64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(sbf_insert_kernel<C>, dim3((uint32_t)blocks), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

template <class C>
hipError_t launch_query(const SeqArgs& a, const Params&)
{
    const uint64_t waves = (round64(a.nk) + C::KPW - 1) / C::KPW;
    const uint64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(sbf_query_kernel<C>, dim3((uint32_t)blocks), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

template <class C>
hipError_t launch_probe(const ProbeArgs& a, const Params&)
{
    uint64_t blocks = (a.n + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(sbf_probe_kernel<C>, dim3((uint32_t)blocks), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

template <int K, int M, int S, int H>
KernelSet spec_set()
{
    using C = Cfg<K, M, S, H>;
    KernelSet ks;
    ks.insert = &launch_insert<C>;
    ks.query = &launch_query<C>;
    ks.probe = &launch_probe<C>;
    ks.specialized = 1;
    return ks;
}

}  // namespace sbf
