// sbf_alpha.hip -- the Super Bloom filter over protein sequences (26 symbols,
// 5 bits) and DNA triplets (64 codons, 6 bits, three bytes per symbol).
//
// Method: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data on
// Modern GPUs" [cuSBF] §IV-A (the three alphabet encodings), §II-B (minimizer
// shard, Findere s-mers), §IV-D/E (insert and query).  The definitions are
// those of the DNA filter with symbols in place of bases: a k-mer of b-bit
// symbols packs first-symbol-most-significant into k*b <= 64 bits, its shard
// is the minimum h_min over its k-m+1 m-mers and its bits are those of its
// k-s+1 s-mers.  A protein symbol is a letter (either case) coded by its
// place in A..Z; a triplet symbol is the codon at bytes 3j..3j+2 coded
// 16 c0 + 4 c1 + c2 from the DNA base codes; anything else is invalid.
//
// Two layouts.  The compile-time parameter sets (the table at the end) run
// the insert and query kernels of sbf_spec.hpp through their text front end:
// 16 symbols per lane packed in registers, sliding windows inside the lane,
// each segment's shard gathered once into LDS.  Any other parameters run this
// file's run-time kernels, and every set runs this file's probe.
//
// Run-time layout (differs from [cuSBF]'s one-k-mer-per-thread tiles): a
// wave64 owns 64 consecutive symbol positions, one per lane, read straight
// from the ASCII text (no packing pass).  The m-mer and s-mer starting at each
// lane are assembled from neighbouring lanes with DPP moves; h_min and h_s are
// then computed once per position, not once per k-mer that contains it.  The
// minimizer of the k-mer starting at lane l is the minimum of h_min over
// lanes l .. l+w-1 (w = k-m+1), and its s-mer bits the OR over lanes
// l .. l+z-1 (z = k-s+1): both are sliding windows across lanes, done by
// doubling (windows of 1, 2, 4, .. lanes, then two overlapping windows).
// Lanes l <= 64-k start a complete k-mer, so one wave step yields 65-k
// k-mers; the rest of the wave is halo.
//
// The run-time insert groups consecutive k-mers of one shard into runs
// (super-k-mers, [cuSBF] §IV-D), ORs each run's masks in an LDS record with
// LDS atomics and issues one global atomic OR per record word, four adjacent
// lanes per record.  The run-time query loads each k-mer's 256-bit shard and
// tests its mask; the wave's answer ballots are appended to a running 64-bit
// word so every store is a whole, aligned answer word.
#include "../../include/sbf.h"
#include "sbf_device.hpp"
#include "sbf_internal.hpp"
#include "sbf_spec.hpp"

namespace sbf {
namespace {

// k-mer starts per wave task: whole answer words, so tasks never share one.
constexpr uint64_t kTask = 2048;

template <int A>
struct Alphabet;

// Protein: byte j, (c | 0x20) - 'a' is 0..25 exactly for the letters.
template <>
struct Alphabet<SBF_ALPHABET_PROTEIN> {
    static constexpr uint32_t B = 5;
    __device__ static __forceinline__ uint32_t code(const char* __restrict__ t, uint64_t j, bool& ok)
    {
        const uint32_t c = (uint32_t)(unsigned char)t[j];
        const uint32_t v = (c | 0x20u) - 0x61u;
        ok = v < 26u;
        return v & 31u;
    }
    // probe symbol j of k-mer i: floor(26 u / 2^64), u the (i k + j + 1)-th
    // SplitMix64 output of the seed
    __device__ static __forceinline__ uint64_t probe(uint64_t seed, uint64_t i, uint32_t k)
    {
        uint64_t x = 0;
        for (uint32_t j = 0; j < k; ++j) {
            const uint64_t u = splitmix_fin(seed + (i * k + j + 1u) * kGolden);
            x = (x << 5) | __umul64hi(u, 26ull);
        }
        return x;
    }
};

// DNA base code ((c >> 1) ^ (c >> 2)) & 3 and its validity: the byte, lower
// cased, must be the letter "acgt"[code].
__device__ __forceinline__ uint32_t base_code(uint32_t c, bool& ok)
{
    const uint32_t v = ((c >> 1) ^ (c >> 2)) & 3u;
    ok = (c | 0x20u) == ((0x74676361u >> (8u * v)) & 0xFFu);
    return v;
}

// Triplet: the codon at bytes 3j .. 3j+2.
template <>
struct Alphabet<SBF_ALPHABET_TRIPLET> {
    static constexpr uint32_t B = 6;
    __device__ static __forceinline__ uint32_t code(const char* __restrict__ t, uint64_t j, bool& ok)
    {
        const unsigned char* p = reinterpret_cast<const unsigned char*>(t) + 3u * j;
        bool o0, o1, o2;
        const uint32_t c0 = base_code(p[0], o0), c1 = base_code(p[1], o1), c2 = base_code(p[2], o2);
        ok = o0 & o1 & o2;
        return (c0 << 4) | (c1 << 2) | c2;
    }
    // the top 6k bits of the (i+1)-th SplitMix64 output, as for DNA
    __device__ static __forceinline__ uint64_t probe(uint64_t seed, uint64_t i, uint32_t k)
    {
        return splitmix_fin(seed + (i + 1u) * kGolden) >> (64u - 6u * k);
    }
};

// Parameters of one kernel instance: compile-time (K, M, S, H nonzero, every
// loop unrolled and every mask index static) or, with zeros, taken from the
// run-time Params (the same code with run-time loops).  A run-time instance
// can still fix H alone (K = M = S = 0, H nonzero), so that the bit-address
// and mask loop unrolls with static word indices.
template <int A, int K, int M, int S, int H>
struct ACfg {
    static constexpr int kAlpha = A;
    static constexpr bool kStatic = K != 0;
    static constexpr uint32_t kK = K, kM = M, kS = S, kH = H;
    __device__ static __forceinline__ uint32_t k(const Params& P) { return K ? (uint32_t)K : P.k; }
    __device__ static __forceinline__ uint32_t m(const Params& P) { return M ? (uint32_t)M : P.m; }
    __device__ static __forceinline__ uint32_t s(const Params& P) { return S ? (uint32_t)S : P.s; }
    __device__ static __forceinline__ uint32_t h(const Params& P) { return H ? (uint32_t)H : P.H; }
};

// h_min of a value below 2^32: (v + G) * C1 = v * C1 + G * C1 (mod 2^64), a
// 32 x 64-bit product.
__device__ __forceinline__ uint64_t hash_min32(uint32_t v)
{
    constexpr uint64_t kGC1 = kGolden * kMulA;
    const uint64_t u = (uint64_t)v * kMulA + kGC1;
    return u ^ (u >> 32);
}

// Every bit of the four masks is set in the shard words w.
__device__ __forceinline__ bool covers(const uint64_t (&w)[4], const uint64_t (&mk)[4])
{
    return ((~w[0] & mk[0]) | (~w[1] & mk[1]) | (~w[2] & mk[2]) | (~w[3] & mk[3])) == 0;
}

// One wave step over symbol positions base .. base+63: for the k-mer that
// starts at this lane, its shard, its four sector masks and whether it is
// to be processed (complete within the wave, every symbol valid, start
// before `end`).
template <class C>
__device__ __forceinline__ bool wave_step(const SeqArgs& a, const Params& P, uint64_t base, uint64_t end,
                                          uint32_t lane, uint32_t& shard, uint64_t (&mk)[4])
{
    using Al = Alphabet<C::kAlpha>;
    const uint32_t k = C::k(P), m = C::m(P), s = C::s(P), H = C::h(P);
    const uint64_t p = base + lane;
    bool ok = false;
    uint32_t sym = 0;
    if (p < a.nsym)
        sym = Al::code(a.text, p, ok);
    const uint64_t V = __ballot(ok);

    // m-mer and s-mer starting here: symbols of lanes l .. l+max(m,s)-1
    uint64_t hm, vs;
    const uint32_t nr = m > s ? m : s;
    uint64_t acc = sym, vm = sym;
    uint32_t t = sym;
    vs = sym;
    for (uint32_t i = 1; i < nr; ++i) {
        t = from_next_lane(t);
        acc = (acc << Al::B) | t;
        if (i + 1u == m)
            vm = acc;
        if (i + 1u == s)
            vs = acc;
    }
    hm = hash_min(vm);
    shard = (uint32_t)window_min(hm, lane_window(k - m + 1u, lane), lane) & a.shard_mask;

    const uint64_t h = hash_s(vs);
    mk[0] = mk[1] = mk[2] = mk[3] = 0;
#pragma unroll
    for (uint32_t j = 0; j < H; ++j) {
        const uint64_t bit = 1ull << bit_addr_rt(h, j, H);
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
            mk[q] |= (j & 3u) == q ? bit : 0ull;
    }
    window_or(mk, lane_window(k - s + 1u, lane), H, lane);

    // k-mer l is valid iff symbols l .. l+k-1 are (bits past lane 63 are 0)
    const uint64_t kv = run_and_rt(V, k);
    return ((kv >> lane) & 1ull) && lane + k <= 64u && p < end;
}

template <class C>
__global__ __launch_bounds__(256) void alpha_insert_kernel(SeqArgs a, Params P)
{
    __shared__ uint64_t rec_mk[4][64][4];
    __shared__ uint32_t rec_sh[4][64];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t S = 65u - C::k(P);  // k-mers per wave step
    const uint32_t nq = C::h(P) < 4u ? C::h(P) : 4u;  // words a record can set
    const uint64_t ntasks = (a.nk + kTask - 1) / kTask;
    const uint64_t wstride = (uint64_t)gridDim.x * 4u;
    const uint64_t le = lane == 63u ? ~0ull : (2ull << lane) - 1ull;  // lanes 0 .. lane
    for (uint64_t task = (uint64_t)blockIdx.x * 4u + wv; task < ntasks; task += wstride) {
        const uint64_t t0 = task * kTask;
        const uint64_t t1 = t0 + kTask < a.nk ? t0 + kTask : a.nk;
        for (uint64_t base = t0; base < t1; base += S) {
            uint32_t shard;
            uint64_t mk[4];
            const bool kv = wave_step<C>(a, P, base, t1, lane, shard, mk);
            // runs: consecutive valid k-mers of one shard
            const uint32_t psh = from_prev_lane(shard);
            const uint32_t pkv = from_prev_lane(kv ? 1u : 0u);
            const bool head = kv && !(pkv && psh == shard);
            const uint64_t HB = __ballot(head);
            const uint32_t nrec = (uint32_t)__popcll(HB);
            if (nrec == 0)
                continue;
            const uint32_t r = (uint32_t)__popcll(HB & le) - 1u;  // this k-mer's run (valid lanes)
            const bool issue = gather_run_quads(mk, nq, kv, __ballot(kv), HB, le, lane);
            reinterpret_cast<ulonglong2*>(rec_mk[wv][lane])[0] = ulonglong2{0, 0};
            reinterpret_cast<ulonglong2*>(rec_mk[wv][lane])[1] = ulonglong2{0, 0};
            wave_lds_sync();
            if (issue) {
#pragma unroll
                for (uint32_t q = 0; q < 4; ++q)
                    if (q < nq)  // every s-mer sets a bit in each word below H
                        __hip_atomic_fetch_or(&rec_mk[wv][r][q], mk[q], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_WAVEFRONT);
                if (head)
                    rec_sh[wv][r] = shard;
            }
            wave_lds_sync();
            // flush: lane -> (record lane/4 + 16 j, word lane & 3); words
            // q >= H of every record are 0 and skipped
            const uint32_t q = lane & 3u;
            if (q < nq)
                for (uint32_t rr = lane >> 2; rr < nrec; rr += 16u) {
                    const uint32_t sh = rec_sh[wv][rr];
                    const uint64_t m = rec_mk[wv][rr][q];
                    atomic_or_u64(a.filter + 4ull * sh + q, m);
                }
            wave_lds_sync();  // the next step rewrites the records
        }
    }
}

template <class C>
__global__ __launch_bounds__(256) void alpha_query_kernel(SeqArgs a, Params P)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t S = 65u - C::k(P);
    const uint64_t ntasks = (a.nk + kTask - 1) / kTask;
    const uint64_t wstride = (uint64_t)gridDim.x * 4u;
    for (uint64_t task = (uint64_t)blockIdx.x * 4u + wv; task < ntasks; task += wstride) {
        const uint64_t t0 = task * kTask;
        const uint64_t t1 = t0 + kTask < a.nk ? t0 + kTask : a.nk;
        uint64_t acc = 0;          // answers not yet stored, first at bit 0
        uint32_t nb = 0;           // how many (< 64)
        uint64_t word = t0 >> 6;   // answer word they belong to
        for (uint64_t base = t0; base < t1; base += S) {
            uint32_t shard;
            uint64_t mk[4];
            bool pres = wave_step<C>(a, P, base, t1, lane, shard, mk);
            if (pres) {
                uint64_t w[4];
                load_shard(a.filter, shard, w);
                pres = covers(w, mk);
            }
            const uint64_t bits = __ballot(pres);  // bits 0 .. S-1
            acc |= bits << nb;
            const uint64_t spill = nb ? bits >> (64u - nb) : 0ull;
            nb += S;
            if (nb >= 64u) {
                if (lane == 0)
                    a.out[word] = acc;
                ++word;
                acc = spill;
                nb -= 64u;
            }
        }
        // the task's last, partial word (never the next task's first)
        if (nb && (word << 6) < t1 && lane == 0)
            a.out[word] = acc;
    }
}

// One random k-mer per lane ([cuSBF] §V-D), every step from its definition.
template <class C>
__global__ __launch_bounds__(256) void alpha_probe_kernel(ProbeArgs a, Params P)
{
    using Al = Alphabet<C::kAlpha>;
    const uint32_t B = Al::B;
    const uint32_t k = C::k(P), m = C::m(P), s = C::s(P), H = C::h(P);
    const uint64_t mmask = (1ull << (B * m)) - 1ull;  // B * m <= 60
    const uint64_t smask = (1ull << (B * s)) - 1ull;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t cnt = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += stride) {
        const uint64_t x = Al::probe(a.seed, i, k);
        uint64_t mn = ~0ull;
#pragma unroll
        for (uint32_t j = 0; j + m <= k; ++j) {
            const uint64_t hm = hash_min((x >> (B * (k - m - j))) & mmask);
            mn = hm < mn ? hm : mn;
        }
        uint64_t w[4];
        load_shard(a.filter, (uint32_t)mn & a.shard_mask, w);
        if constexpr (C::kStatic) {
            // compile-time H: test the k-mer's bits one by one (a shift each)
            uint32_t hit = 1u;
#pragma unroll
            for (uint32_t j = 0; j + s <= k; ++j) {
                const uint64_t h = hash_s((x >> (B * (k - s - j))) & smask);
#pragma unroll
                for (uint32_t t = 0; t < H; ++t)
                    hit &= (uint32_t)(w[t & 3u] >> bit_addr_rt(h, t, H));
            }
            cnt += hit & 1u;
        } else {
            uint64_t mk[4] = {0, 0, 0, 0};
            for (uint32_t j = 0; j + s <= k; ++j) {
                const uint64_t h = hash_s((x >> (B * (k - s - j))) & smask);
                for (uint32_t t = 0; t < H; ++t) {
                    const uint64_t bit = 1ull << bit_addr_rt(h, t, H);
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q)
                        mk[q] |= (t & 3u) == q ? bit : 0ull;
                }
            }
            cnt += covers(w, mk) ? 1u : 0u;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

uint32_t task_blocks(uint64_t nk)
{
    const uint64_t tasks = (nk + kTask - 1) / kTask;
    uint64_t b = (tasks + 3) / 4;
    if (b > 16384)
        b = 16384;
    return (uint32_t)(b ? b : 1);
}

template <class C>
hipError_t alpha_insert(const SeqArgs& a, const Params& P)
{
    if (a.nk == 0)
        return hipSuccess;
    hipLaunchKernelGGL(alpha_insert_kernel<C>, dim3(task_blocks(a.nk)), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

template <class C>
hipError_t alpha_query(const SeqArgs& a, const Params& P)
{
    if (a.nk == 0)
        return hipSuccess;
    hipLaunchKernelGGL(alpha_query_kernel<C>, dim3(task_blocks(a.nk)), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

template <class C>
hipError_t alpha_probe(const ProbeArgs& a, const Params& P)
{
    if (a.n == 0)
        return hipSuccess;
    uint64_t b = (a.n + 255) / 256;
    if (b > 8192)
        b = 8192;
    hipLaunchKernelGGL(alpha_probe_kernel<C>, dim3((uint32_t)b), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

template <class C>
KernelSet make_alpha()
{
    KernelSet ks;
    ks.insert = &alpha_insert<C>;
    ks.query = &alpha_query<C>;
    ks.probe = &alpha_probe<C>;
    ks.specialized = C::kStatic ? 1 : 0;
    return ks;
}

// Compile-time instances: the insert and query of the DNA kernels
// (sbf_spec.hpp: 16 symbols per lane, runs gathered once per segment) read
// the text through their text front end; the probe is this file's.
template <int A, int K, int M, int S, int H>
KernelSet make_alpha_spec()
{
    using C = Cfg<K, M, S, H, 16, (int)A>;
    KernelSet ks;
    ks.insert = &launch_insert<C>;
    ks.query = &launch_query<C>;
    ks.probe = &alpha_probe<ACfg<A, K, M, S, H>>;
    ks.specialized = 1;
    return ks;
}

// The default protein (k=12, m=6, s=10, H=4) and triplet (k=10, m=5, s=8,
// H=4) parameters and one neighbour of each.
struct AlphaEntry {
    uint32_t alpha, k, m, s, H;
    KernelSet (*make)();
};
constexpr uint32_t kP = SBF_ALPHABET_PROTEIN, kT = SBF_ALPHABET_TRIPLET;
const AlphaEntry kAlphaTable[] = {
    {kP, 12, 6, 10, 4, &make_alpha_spec<kP, 12, 6, 10, 4>},
    {kP, 9, 4, 7, 3, &make_alpha_spec<kP, 9, 4, 7, 3>},
    {kT, 10, 5, 8, 4, &make_alpha_spec<kT, 10, 5, 8, 4>},
    {kT, 7, 3, 7, 2, &make_alpha_spec<kT, 7, 3, 7, 2>},
};

// Run-time kernels of one alphabet, with H fixed at compile time for
// 1 <= H <= 16 and taken at run time above.
template <uint32_t A>
KernelSet alpha_runtime(uint32_t H)
{
    switch (H) {
    case 1: return make_alpha<ACfg<A, 0, 0, 0, 1>>();
    case 2: return make_alpha<ACfg<A, 0, 0, 0, 2>>();
    case 3: return make_alpha<ACfg<A, 0, 0, 0, 3>>();
    case 4: return make_alpha<ACfg<A, 0, 0, 0, 4>>();
    case 5: return make_alpha<ACfg<A, 0, 0, 0, 5>>();
    case 6: return make_alpha<ACfg<A, 0, 0, 0, 6>>();
    case 7: return make_alpha<ACfg<A, 0, 0, 0, 7>>();
    case 8: return make_alpha<ACfg<A, 0, 0, 0, 8>>();
    case 9: return make_alpha<ACfg<A, 0, 0, 0, 9>>();
    case 10: return make_alpha<ACfg<A, 0, 0, 0, 10>>();
    case 11: return make_alpha<ACfg<A, 0, 0, 0, 11>>();
    case 12: return make_alpha<ACfg<A, 0, 0, 0, 12>>();
    case 13: return make_alpha<ACfg<A, 0, 0, 0, 13>>();
    case 14: return make_alpha<ACfg<A, 0, 0, 0, 14>>();
    case 15: return make_alpha<ACfg<A, 0, 0, 0, 15>>();
    case 16: return make_alpha<ACfg<A, 0, 0, 0, 16>>();
    default: return make_alpha<ACfg<A, 0, 0, 0, 0>>();
    }
}

}  // namespace

KernelSet alpha_kernels(const Params& P)
{
    for (const AlphaEntry& e : kAlphaTable)
        if (e.alpha == P.alpha && e.k == P.k && e.m == P.m && e.s == P.s && e.H == P.H)
            return e.make();
    return P.alpha == SBF_ALPHABET_TRIPLET ? alpha_runtime<kT>(P.H) : alpha_runtime<kP>(P.H);
}

}  // namespace sbf
