// sbf_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// hash functions, bit addressing, packed-sequence windows and validity.
//
// Method: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on
// Modern GPUs" [cuSBF].  Hash choices are fixed in include/sbf.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbf {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;  // 2^64 / golden ratio
constexpr uint64_t kMulA = 0xBF58476D1CE4E5B9ull;    // SplitMix64 multipliers
constexpr uint64_t kMulB = 0x94D049BB133111EBull;

// [cuSBF] §IV-G role-specialized hashing: one multiplicative mix for the
// minimizer (folded so the low shard bits see every base) ...
__device__ __forceinline__ uint64_t hash_min(uint64_t v)
{
    const uint64_t u = (v + kGolden) * kMulA;
    return u ^ (u >> 32);
}

// ... and a stronger mix for the s-mers (SplitMix64 finalizer of v + G).
__device__ __forceinline__ uint64_t splitmix_fin(uint64_t z)
{
    z = (z ^ (z >> 30)) * kMulA;
    z = (z ^ (z >> 27)) * kMulB;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t hash_s(uint64_t v) { return splitmix_fin(v + kGolden); }

// Per-hash-index salt of the H > 10 fallback: the t-th SplitMix64 output of
// seed 0, i.e. the finalizer of (t+1) * G.
__host__ __device__ constexpr uint64_t salt_of(uint32_t t)
{
    uint64_t z = (uint64_t)(t + 1u) * kGolden;
    z = (z ^ (z >> 30)) * kMulA;
    z = (z ^ (z >> 27)) * kMulB;
    return z ^ (z >> 31);
}

// [cuSBF] §IV-G bit-slicing (H <= 10) and golden-ratio salted fallback.
template <int H>
__device__ __forceinline__ uint32_t bit_addr(uint64_t h, int t)
{
    if constexpr (H <= 10) {
        constexpr int width = 64 / H;
        return (uint32_t)(h >> (t * width)) & 63u;
    } else {
        return (uint32_t)((h * salt_of((uint32_t)t)) >> 58);
    }
}

__device__ __forceinline__ uint32_t bit_addr_rt(uint64_t h, uint32_t t, uint32_t H)
{
    if (H <= 10)
        return (uint32_t)(h >> (t * (64u / H))) & 63u;
    return (uint32_t)((h * salt_of(t)) >> 58);
}

// Wide-block variant: 9-bit address into a 512-bit block, slices of width
// floor(64/H) for H <= 7, else the top 9 bits of h * salt_t.
template <int H>
__device__ __forceinline__ uint32_t bit_addr_wide(uint64_t h, int t)
{
    if constexpr (H <= 7) {
        constexpr int width = 64 / H;
        return (uint32_t)(h >> (t * width)) & 511u;
    } else {
        return (uint32_t)((h * salt_of((uint32_t)t)) >> 55);
    }
}

__device__ __forceinline__ uint32_t bit_addr_wide_rt(uint64_t h, uint32_t t, uint32_t H)
{
    if (H <= 7)
        return (uint32_t)(h >> (t * (64u / H))) & 511u;
    return (uint32_t)((h * salt_of(t)) >> 55);
}

// Four ASCII bytes (first base in the low byte) -> one code byte with the
// first base in its top two bits, and four validity bits (bit j = byte j).
__device__ __forceinline__ void encode_dword(uint32_t w, uint32_t& code_byte, uint32_t& valid4)
{
    // A=0x41 C=0x43 G=0x47 T=0x54 (and lower case): ((c>>1)^(c>>2))&3 = 0,1,2,3
    const uint32_t c = ((w >> 1) ^ (w >> 2)) & 0x03030303u;
    // c0 + c1<<8 + c2<<16 + c3<<24 times 2^30+2^20+2^10+1 puts c0..c3 at bits
    // 30,28,26,24 with every cross term below bit 24 and no carry into it
    code_byte = (c * 0x40100401u) >> 24;
    // valid iff the byte, lower-cased, is the letter its code stands for
    const uint32_t expect = __builtin_amdgcn_perm(0x74676361u, 0x74676361u, c);  // "acgt" by code
    const uint32_t diff = (w | 0x20202020u) ^ expect;
    // exact zero-byte flags: high bit of byte j set iff byte j of diff is 0
    const uint32_t t = (diff & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
    const uint32_t z = ~(t | diff | 0x7F7F7F7Fu);
    // flags at bits 7,15,23,31 -> bits 21..24 via one multiply
    valid4 = ((((z >> 7) & 0x01010101u) * 0x00204081u) >> 21) & 0xFu;
}

// Top 32 bits of the 64-bit value (a:b) shifted left by r, 0 <= r < 32.
__device__ __forceinline__ uint32_t funnel_hi(uint32_t a, uint32_t b, uint32_t r)
{
    return r == 0 ? a : (uint32_t)((((uint64_t)a << 32) | b) >> (32 - r));
}

// 64 bits of the packed base stream D starting at base i (i compile-time
// after unrolling): bases i..i+31, first base in the top bits.
template <int NDW>
__device__ __forceinline__ uint64_t stream_window(const uint32_t (&D)[NDW], int i)
{
    const int a = i >> 4;
    const uint32_t r = 2u * (uint32_t)(i & 15);
    const uint32_t hi = funnel_hi(D[a], D[a + 1], r);
    const uint32_t lo = funnel_hi(D[a + 1], D[a + 2], r);
    return ((uint64_t)hi << 32) | lo;
}

// Value of the n-base window whose first base is the top of `win` (n <= 32).
__device__ __forceinline__ uint64_t top_bases(uint64_t win, int n)
{
    return n >= 32 ? win : (win >> (64 - 2 * n));
}

// Read word idx of a uint32 array, 0 past its end.
__device__ __forceinline__ uint32_t ld_or0(const uint32_t* __restrict__ a, uint64_t n, uint64_t idx)
{
    return idx < n ? a[idx] : 0u;
}

// Validity bits of bases p0 .. p0+63 (bit i = base p0+i), p0 % 16 == 0.
__device__ __forceinline__ uint64_t valid_window64(const uint32_t* __restrict__ valid, uint64_t nvw, uint64_t p0)
{
    const uint64_t w = p0 >> 5;
    const uint32_t off = (uint32_t)(p0 & 31);
    const uint64_t v01 = (uint64_t)ld_or0(valid, nvw, w) | ((uint64_t)ld_or0(valid, nvw, w + 1) << 32);
    uint64_t win = v01 >> off;
    if (off)
        win |= (uint64_t)ld_or0(valid, nvw, w + 2) << (64 - off);
    return win;
}

// Bit i of the result is 1 iff bits i .. i+k-1 of v are all 1 (k <= 32).
template <int KK>
__device__ __forceinline__ uint64_t run_and(uint64_t v)
{
    uint64_t a[6];
    a[0] = v;
#pragma unroll
    for (int j = 1; j < 6; ++j)
        a[j] = a[j - 1] & (a[j - 1] >> (1 << (j - 1)));
    uint64_t r = ~0ull;
    int pos = 0;
#pragma unroll
    for (int j = 5; j >= 0; --j) {
        if (KK & (1 << j)) {
            r &= a[j] >> pos;
            pos += 1 << j;
        }
    }
    return r;
}

__device__ __forceinline__ uint64_t run_and_rt(uint64_t v, uint32_t kk)
{
    uint64_t r = ~0ull;
    uint32_t pos = 0;
    uint64_t a = v;
    uint64_t levels[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        levels[j] = a;
        a = a & (a >> (1 << j));
    }
#pragma unroll
    for (int j = 5; j >= 0; --j) {
        if (kk & (1u << j)) {
            r &= levels[j] >> pos;
            pos += 1u << j;
        }
    }
    return r;
}

__device__ __forceinline__ void atomic_or_u64(uint64_t* p, uint64_t v)
{
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Load one 256-bit shard (two 128-bit loads).
__device__ __forceinline__ void load_shard(const uint64_t* __restrict__ filter, uint64_t shard, uint64_t (&w)[4])
{
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(filter + 4 * shard);
    const ulonglong2 a = p[0];
    const ulonglong2 b = p[1];
    w[0] = a.x;
    w[1] = a.y;
    w[2] = b.x;
    w[3] = b.y;
}

// Value of lane l+1 in lane l (lane 63 receives 0): one DPP wave_shl:1 move
// per 32-bit half, no LDS traffic.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v)
{
    // bound_ctrl: lane 63 reads 0 instead of keeping an old value, so no copy
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x130, 0xF, 0xF, true);
}

// Value of lane l-1 in lane l (lane 0 receives 0): DPP wave_shr:1.
__device__ __forceinline__ uint32_t from_prev_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x138, 0xF, 0xF, true);
}

__device__ __forceinline__ uint64_t from_next_lane(uint64_t v)
{
    return ((uint64_t)from_next_lane((uint32_t)(v >> 32)) << 32) | from_next_lane((uint32_t)v);
}

// Raw buffer over the 32-bit words [w0, n) of an array, w0 wave-uniform: a
// read past the end returns 0 through the buffer range check, so lane loads
// need no bounds branches.  Descriptor word 3: 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t word_buffer(const uint32_t* a, uint64_t n, uint64_t w0)
{
    const uint64_t b = w0 < n ? w0 : n;
    const uint64_t bytes = (n - b) * 4ull;
    const uint32_t nrec = bytes < 0xFFFFFFFFull ? (uint32_t)bytes : 0xFFFFFFFFu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a + b), (short)0, (int)nrec, 0x00020000);
}

// Plan of a minimum or an OR over lanes l .. l+n-1 (1 <= n <= 64, n
// wave-uniform): doubling steps over spans 1, 2, 4, ... while twice the span
// still fits in n (2^levels <= n), then one step over the remaining
// n - 2^levels lanes.  Made once per kernel or step from n, so the steps
// themselves are straight-line code with one uniform branch each (none when
// n is a compile-time constant).  Lanes past 63 read garbage; only halo
// lanes look there.
struct LaneWindow {
    uint32_t levels;    // doubling steps (spans 1 .. 2^(levels-1))
    uint32_t rem;       // lanes of the last step, 0 for none
    uint32_t rem_addr;  // ds_bpermute byte address of lane l + rem
};

__device__ __forceinline__ LaneWindow lane_window(uint32_t n, uint32_t lane)
{
    LaneWindow w;
    w.levels = 31u - (uint32_t)__builtin_clz(n);
    w.rem = n - (1u << w.levels);
    w.rem_addr = (lane + w.rem) << 2;
    return w;
}

// Value of the lane whose ds_bpermute byte address is addr.
__device__ __forceinline__ uint64_t lane_at(uint64_t v, uint32_t addr)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)addr, (int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// min over lanes l .. l+n-1 of v
__device__ __forceinline__ uint64_t window_min(uint64_t v, const LaneWindow& W, uint32_t lane)
{
    if (W.levels >= 1u) {
        const uint64_t o = from_next_lane(v);  // span 1 by DPP
        v = o < v ? o : v;
    }
#pragma unroll
    for (uint32_t j = 1; j < 6; ++j)
        if (W.levels > j) {
            const uint64_t o = lane_at(v, (lane + (1u << j)) << 2);
            v = o < v ? o : v;
        }
    if (W.rem) {
        const uint64_t o = lane_at(v, W.rem_addr);
        v = o < v ? o : v;
    }
    return v;
}

// OR over lanes l .. l+n-1 of the four sector masks (words q >= H stay 0)
__device__ __forceinline__ void window_or(uint64_t (&mk)[4], const LaneWindow& W, uint32_t H, uint32_t lane)
{
    const uint32_t nq = H < 4u ? H : 4u;
    if (W.levels >= 1u) {
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
            if (q < nq)
                mk[q] |= from_next_lane(mk[q]);
    }
#pragma unroll
    for (uint32_t j = 1; j < 6; ++j)
        if (W.levels > j) {
            const uint32_t addr = (lane + (1u << j)) << 2;
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q)
                if (q < nq)
                    mk[q] |= lane_at(mk[q], addr);
        }
    if (W.rem) {
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
            if (q < nq)
                mk[q] |= lane_at(mk[q], W.rem_addr);
    }
}

// Before the k-mers of a run OR their masks into the run's LDS record: a
// k-mer takes the masks of lane l+1 and then of the pair at lane l+2 where
// its run goes on that far (DPP moves), and only the k-mers at offsets 0, 4,
// 8 ... from their run's head go on to OR into the record.  A quarter as many
// lanes then meet on each record, whose LDS atomics serialize.  KV and HB are
// the wave's ballots of valid k-mers and run heads, le the mask of lanes
// 0 .. lane; words q >= nq are left alone.  Returns whether this lane ORs.
__device__ __forceinline__ bool gather_run_quads(uint64_t (&mk)[4], uint32_t nq, bool kv, uint64_t KV, uint64_t HB,
                                                 uint64_t le, uint32_t lane)
{
    const uint64_t cont = KV & ~HB;  // valid k-mers that continue the run of lane l-1
    const bool same1 = kv && lane < 63u && ((cont >> (lane + 1u)) & 1ull);
    const bool same2 = same1 && lane < 62u && ((cont >> (lane + 2u)) & 1ull);
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q)
        if (q < nq) {
            const uint64_t n1 = from_next_lane(mk[q]);
            mk[q] |= same1 ? n1 : 0ull;
            const uint64_t n2 = from_next_lane(from_next_lane(mk[q]));
            mk[q] |= same2 ? n2 : 0ull;
        }
    const uint32_t hp = 63u - (uint32_t)__builtin_clzll((HB & le) | 1ull);  // this run's head lane
    return kv && ((lane - hp) & 3u) == 0u;
}

// LDS written by some lanes of this wave becomes visible to all its lanes.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sbf
