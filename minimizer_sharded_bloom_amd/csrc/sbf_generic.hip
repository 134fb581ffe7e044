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
// separators).  One lane per 32 bases: two 16-byte loads, two code words and
// one validity word, four bases per 32-bit SIMD-within-a-register step.
// ---------------------------------------------------------------------------

// 16 bases (four dwords) -> one code word (first base in bits 31..30) and 16
// validity bits.
__device__ __forceinline__ void encode16(uint4 q, uint32_t& code, uint32_t& val)
{
    uint32_t b0, b1, b2, b3, v0, v1, v2, v3;
    encode_dword(q.x, b0, v0);
    encode_dword(q.y, b1, v1);
    encode_dword(q.z, b2, v2);
    encode_dword(q.w, b3, v3);
    code = (b0 << 24) | (b1 << 16) | (b2 << 8) | b3;
    val = v0 | (v1 << 4) | (v2 << 8) | (v3 << 12);
}

__device__ __forceinline__ uint4 load16_tail(const char* __restrict__ ascii, uint64_t base, uint64_t len)
{
    uint32_t q[4] = {0, 0, 0, 0};
    for (int j = 0; j < 16 && base + j < len; ++j)
        q[j >> 2] |= (uint32_t)(unsigned char)ascii[base + j] << (8 * (j & 3));
    return make_uint4(q[0], q[1], q[2], q[3]);
}

__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ ascii, uint64_t len,
                                                   uint32_t* __restrict__ codes, uint32_t* __restrict__ valid,
                                                   uint64_t ncw, uint64_t nvw, int aligned16)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;  // validity word index
    if (i >= nvw)
        return;
    const uint64_t base = 32 * i;
    uint4 q0, q1;
    if (base + 32 <= len && aligned16) {
        const uint4* p = reinterpret_cast<const uint4*>(ascii + base);
        q0 = p[0];
        q1 = p[1];
    } else {
        q0 = load16_tail(ascii, base, len);
        q1 = load16_tail(ascii, base + 16, len);
    }
    uint32_t c0, c1, v0, v1;
    encode16(q0, c0, v0);
    encode16(q1, c1, v1);
    uint32_t val = v0 | (v1 << 16);
    if (base + 32 > len)  // bases past len are invalid (their zero bytes already are)
        val &= (uint32_t)((1ull << (len - base)) - 1ull);
    codes[2 * i] = c0;
    if (2 * i + 1 < ncw)
        codes[2 * i + 1] = c1;
    valid[i] = val;
}

hipError_t launch_pack(const char* ascii, uint64_t len, uint32_t* codes, uint32_t* valid, hipStream_t st)
{
    if (len == 0)
        return hipSuccess;
    const uint64_t ncw = (len + 15) / 16;
    const uint64_t nvw = (len + 31) / 32;
    const int aligned = ((uintptr_t)ascii & 15u) == 0;
    const uint64_t blocks = (nvw + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, ascii, len, codes, valid, ncw, nvw,
                       aligned);
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

__global__ __launch_bounds__(256) void reads_remap_kernel(const uint64_t* __restrict__ bits, uint64_t nbw, uint64_t n,
                                                          uint64_t stride, uint32_t nkr, uint32_t rch,
                                                          uint32_t* __restrict__ out)
{
    const uint64_t total = n * rch;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += step) {
        const uint64_t r = g / rch, j = g - r * rch;
        const uint64_t b = r * stride + 32u * j;  // bit of the read's k-mer 32j
        const uint64_t w = b >> 6;
        const uint32_t sh = (uint32_t)(b & 63u);
        uint64_t v = bits[w] >> sh;
        if (sh > 32u && w + 1 < nbw)
            v |= bits[w + 1] << (64u - sh);
        const uint32_t left = nkr - 32u * (uint32_t)j;
        out[g] = (uint32_t)v & (left >= 32u ? 0xFFFFFFFFu : (1u << left) - 1u);
    }
}

hipError_t launch_reads_remap(const uint64_t* bits, uint64_t nbw, uint64_t n, uint64_t stride, uint32_t nkr,
                              uint32_t rch, uint32_t* out, hipStream_t st)
{
    const uint64_t total = n * rch;
    if (total == 0)
        return hipSuccess;
    uint64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(reads_remap_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, bits, nbw, n, stride, nkr, rch,
                       out);
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

// Words per shard: 8 for the wide-block variant (kind 2), else 4.
__device__ __forceinline__ uint32_t shard_words(const Params& P) { return P.kind == 2 ? 8u : 4u; }

// Bits of one hash value: word t mod 4 (sectorized kinds) or, for the wide
// variant, bit a mod 64 of word a / 64 for the 9-bit address a
// ([cuSBF] §V-D, the CPU reference's whole-block addressing).
__device__ __forceinline__ void hash_bits(uint64_t h, const Params& P, uint64_t (&mk)[8])
{
    for (uint32_t t = 0; t < P.H; ++t) {
        if (P.kind == 2) {
            const uint32_t a = bit_addr_wide_rt(h, t, P.H);
            const uint64_t bit = 1ull << (a & 63u);
#pragma unroll
            for (uint32_t w = 0; w < 8; ++w)
                mk[w] |= (a >> 6) == w ? bit : 0ull;
        } else {
            const uint64_t bit = 1ull << bit_addr_rt(h, t, P.H);
#pragma unroll
            for (uint32_t w = 0; w < 4; ++w)
                mk[w] |= (t & 3u) == w ? bit : 0ull;
        }
    }
}

__device__ __forceinline__ void kmer_masks(uint64_t x, const Params& P, uint64_t (&mk)[8])
{
#pragma unroll
    for (int w = 0; w < 8; ++w)
        mk[w] = 0;
    if (P.kind == 1) {
        hash_bits(hash_s(hash_s(x)), P, mk);
        return;
    }
    for (uint32_t j = 0; j + P.s <= P.k; ++j)
        hash_bits(hash_s(sub_rt(x, P.k, j, P.s)), P, mk);
}

// One k-mer per lane, 64 k-mers per wave step.  Each lane stages its shard
// and masks in LDS; then W adjacent lanes (W = words per shard) OR the W
// words of one record into the filter in one instruction, which the memory
// system merges into one request per k-mer instead of W.
__global__ __launch_bounds__(256) void generic_insert_kernel(SeqArgs a, Params P)
{
    __shared__ uint32_t rec_idx[4][64];
    __shared__ uint64_t rec_words[4][64][8];
    const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
    const uint32_t W = shard_words(P), lw = W == 8 ? 3u : 2u;
    const uint64_t nk_pad = (a.nk + 63) & ~63ull;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t p0 = (uint64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63u); p0 < nk_pad; p0 += stride) {
        const uint64_t p = p0 + lane;
        uint64_t mk[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t sh = 0;
        if (p < a.nk && kmer_valid_at(a.valid, a.nvw, p, P.k)) {
            const uint64_t x = kmer_at(a.codes, a.ncw, p, P.k);
            sh = kmer_shard(x, P, a.shard_mask);
            kmer_masks(x, P, mk);
        }
        rec_idx[wv][lane] = sh;
        for (int q = 0; q < 8; ++q)
            rec_words[wv][lane][q] = mk[q];
        wave_lds_sync();
        for (uint32_t j = 0; j < W; ++j) {
            const uint32_t r = (lane >> lw) + (64u >> lw) * j, q = lane & (W - 1u);
            const uint64_t m = rec_words[wv][r][q];
            if (m)
                atomic_or_u64(a.filter + (uint64_t)W * rec_idx[wv][r] + q, m);
        }
        wave_lds_sync();  // the next step overwrites the records
    }
}

// Every query mask bit must be set in the shard (W words).
__device__ __forceinline__ bool shard_has(const uint64_t* __restrict__ filter, uint32_t sh, const uint64_t (&mk)[8],
                                          uint32_t W)
{
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(filter + (uint64_t)W * sh);
    bool ok = true;
    for (uint32_t i = 0; i < W / 2; ++i) {
        const ulonglong2 v = p[i];
        ok &= ((v.x & mk[2 * i]) == mk[2 * i]) & ((v.y & mk[2 * i + 1]) == mk[2 * i + 1]);
    }
    return ok;
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
            uint64_t mk[8];
            kmer_masks(x, P, mk);
            pres = shard_has(a.filter, kmer_shard(x, P, a.shard_mask), mk, shard_words(P));
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
        uint64_t mk[8];
        kmer_masks(x, P, mk);
        cnt += shard_has(a.filter, kmer_shard(x, P, a.shard_mask), mk, shard_words(P));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

// FPR probe of a Super Bloom filter with run-time k, m, s ([cuSBF] §V-D:
// random k-mers, each answered on its own).  HC > 0 fixes H at compile time,
// so each s-mer's bits go to static words; HC = 0 takes H from P.  The m-mers
// and s-mers are cut from the k-mer by a running 2-bit shift, last first, so
// no window needs a shift by a run-time amount.
template <int HC>
__global__ __launch_bounds__(256) void sbf_probe_rt_kernel(ProbeArgs a, Params P)
{
    const uint32_t k = P.k, m = P.m, s = P.s, H = HC ? (uint32_t)HC : P.H;
    const uint64_t mmask = m >= 32u ? ~0ull : (1ull << (2u * m)) - 1ull;
    const uint64_t smask = s >= 32u ? ~0ull : (1ull << (2u * s)) - 1ull;
    const uint32_t w = k - m + 1u, z = k - s + 1u;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t cnt = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += stride) {
        const uint64_t x = splitmix_fin(a.seed + (i + 1) * kGolden) >> (64 - 2 * k);
        uint64_t mn = ~0ull, y = x;
        for (uint32_t j = 0; j < w; ++j, y >>= 2) {
            const uint64_t h = hash_min(y & mmask);
            mn = h < mn ? h : mn;
        }
        uint64_t mk[4] = {0, 0, 0, 0};
        y = x;
        for (uint32_t j = 0; j < z; ++j, y >>= 2) {
            const uint64_t h = hash_s(y & smask);
            if constexpr (HC > 0) {
#pragma unroll
                for (int t = 0; t < HC; ++t)
                    mk[t & 3] |= 1ull << bit_addr<HC>(h, t);
            } else {
                for (uint32_t t0 = 0; t0 < H; t0 += 4u) {
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q)
                        if (t0 + q < H)
                            mk[q] |= 1ull << bit_addr_rt(h, t0 + q, H);
                }
            }
        }
        uint64_t sw[4];
        load_shard(a.filter, (uint32_t)mn & a.shard_mask, sw);
        cnt += ((~sw[0] & mk[0]) | (~sw[1] & mk[1]) | (~sw[2] & mk[2]) | (~sw[3] & mk[3])) == 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63u) == 0 && cnt)
        atomicAdd(a.hits, (unsigned long long)cnt);
}

// ---------------------------------------------------------------------------
// Run-time sliding kernels of the Super Bloom filter (any k, m, s, H that has
// no compiled set).  A wave step covers 64 consecutive positions, one per
// lane: lane l reads the packed bases p .. p+31 (p = base + l) from the code
// words and hashes the m-mer and the s-mer starting at p once; the k-mer
// starting at p takes the minimum h_min over lanes l .. l+w-1 (its w = k-m+1
// m-mers, [cuSBF] Algorithm 1) and the OR of the s-mer sector masks over
// lanes l .. l+z-1 (its z = k-s+1 s-mers), both by cross-lane doubling.  The
// lanes l < E = 65 - max(w, z) start a complete k-mer, so one step yields E
// k-mers and the rest of the wave is halo.  Every position is hashed once
// per step instead of w + z times per k-mer as in the per-k-mer kernels.
// ---------------------------------------------------------------------------

// k-mer starts per wave task: whole answer words, so tasks never share one.
constexpr uint64_t kSlideTask = 2048;

// What a wave keeps for one task of the sliding kernels: raw buffers over the
// code and validity words from the task's first ones (a read past the end of
// the sequence returns 0 through the buffer range check, so lane loads need
// no bounds branches), and the plans of the minimizer's and the Findere
// mask's cross-lane windows.
struct SlideTask {
    __amdgpu_buffer_rsrc_t rc, rv;
    uint64_t wc0, wv0;  // first code and validity word of the buffers
    LaneWindow wm, wz;  // over w = k-m+1 and z = k-s+1 lanes

    __device__ __forceinline__ SlideTask(const SeqArgs& a, const Params& P, uint64_t t0, uint32_t lane)
        : rc(word_buffer(a.codes, a.ncw, t0 >> 4)), rv(word_buffer(a.valid, a.nvw, t0 >> 5)), wc0(t0 >> 4),
          wv0(t0 >> 5), wm(lane_window(P.k - P.m + 1u, lane)), wz(lane_window(P.k - P.s + 1u, lane))
    {
    }
};

// The words a lane reads for one wave step: code words holding its bases
// p .. p+31 and validity words holding bits p .. p+63.  Loaded one step
// ahead, so the loads of step i+1 are in flight while step i computes.
struct SlideWords {
    uint32_t d0, d1, d2, v0, v1, v2;
};

__device__ __forceinline__ SlideWords slide_load(const SlideTask& T, uint64_t base, uint32_t lane)
{
    SlideWords W;
    const uint32_t o = ((uint32_t)((base >> 4) - T.wc0) + (((uint32_t)(base & 15u) + lane) >> 4)) * 4u;
    W.d0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rc, (int)o, 0, 0);
    W.d1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rc, (int)(o + 4u), 0, 0);
    W.d2 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rc, (int)(o + 8u), 0, 0);
    const uint32_t vo = ((uint32_t)((base >> 5) - T.wv0) + (((uint32_t)(base & 31u) + lane) >> 5)) * 4u;
    W.v0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rv, (int)vo, 0, 0);
    W.v1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rv, (int)(vo + 4u), 0, 0);
    W.v2 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(T.rv, (int)(vo + 8u), 0, 0);
    return W;
}

// Shard key (low 32 bits of the minimizer hash) and sector masks of the k-mer
// starting at this lane's position, from the step's words; true if it is to
// be processed (a start lane, before `end`, every base valid).  HC > 0 fixes
// H at compile time (the bit-address loop unrolls); HC = 0 takes it from P.
template <int HC>
__device__ __forceinline__ bool slide_step(const Params& P, const SlideTask& T, const SlideWords& D, uint64_t base,
                                           uint64_t end, uint32_t lane, uint32_t E, uint32_t& key, uint64_t (&mk)[4])
{
    const uint32_t k = P.k, m = P.m, s = P.s, H = HC ? (uint32_t)HC : P.H;
    const uint64_t p = base + lane;
    // bases p .. p+31, first in the top bits
    const uint32_t r = 2u * (uint32_t)(p & 15u);
    const uint64_t win = ((uint64_t)funnel_hi(D.d0, D.d1, r) << 32) | funnel_hi(D.d1, D.d2, r);
    // validity bits p .. p+63
    const uint32_t voff = ((uint32_t)(base & 31u) + lane) & 31u;
    const uint64_t vwin = ((uint64_t)__builtin_amdgcn_alignbit(D.v2, D.v1, voff) << 32) |
                          __builtin_amdgcn_alignbit(D.v1, D.v0, voff);
    const uint64_t need = k >= 64u ? ~0ull : ((1ull << k) - 1ull);

    const uint64_t vm = m >= 32u ? win : win >> (64u - 2u * m);
    const uint64_t vs = s >= 32u ? win : win >> (64u - 2u * s);
    key = (uint32_t)window_min(hash_min(vm), T.wm, lane);
    const uint64_t h = hash_s(vs);
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q)
        mk[q] = 0;
    if constexpr (HC > 0) {
#pragma unroll
        for (int t = 0; t < HC; ++t)
            mk[t & 3] |= 1ull << bit_addr<HC>(h, t);
    } else {
        for (uint32_t t0 = 0; t0 < H; t0 += 4u) {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q)
                if (t0 + q < H)
                    mk[q] |= 1ull << bit_addr_rt(h, t0 + q, H);
        }
    }
    window_or(mk, T.wz, H, lane);
    return lane < E && p < end && (vwin & need) == need;
}

// Step length: E = 65 - max(w, z) k-mers per wave step.
__device__ __forceinline__ uint32_t slide_yield(const Params& P)
{
    const uint32_t w = P.k - P.m + 1u, z = P.k - P.s + 1u;
    return 65u - (w > z ? w : z);
}

// Insert: consecutive valid k-mers of one shard key within a step form a run
// ([cuSBF] §IV-D super-k-mers); each run ORs its k-mers' masks into an LDS
// record with LDS atomics, and four adjacent lanes OR one record's words
// into the filter (one merged request per run).
template <int HC>
__global__ __launch_bounds__(256) void slide_insert_kernel(SeqArgs a, Params P)
{
    __shared__ uint64_t rec_mk[4][64][4];
    __shared__ uint32_t rec_sh[4][64];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t E = slide_yield(P);
    const uint32_t H = HC ? (uint32_t)HC : P.H, nq = H < 4u ? H : 4u;  // words a record can set
    const uint64_t ntasks = (a.nk + kSlideTask - 1) / kSlideTask;
    const uint64_t wstride = (uint64_t)gridDim.x * 4u;
    const uint64_t le = lane == 63u ? ~0ull : (2ull << lane) - 1ull;  // lanes 0 .. lane
    for (uint64_t task = (uint64_t)blockIdx.x * 4u + wv; task < ntasks; task += wstride) {
        const uint64_t t0 = task * kSlideTask;
        const uint64_t t1 = t0 + kSlideTask < a.nk ? t0 + kSlideTask : a.nk;
        const SlideTask T(a, P, t0, lane);
        SlideWords D = slide_load(T, t0, lane);
        for (uint64_t base = t0; base < t1; base += E) {
            const SlideWords cur = D;
            D = slide_load(T, base + E, lane);  // the next step's words (past the task: unused)
            uint32_t key;
            uint64_t mk[4];
            const bool kv = slide_step<HC>(P, T, cur, base, t1, lane, E, key, mk);
            const uint32_t pkey = from_prev_lane(key);
            const uint32_t pkv = from_prev_lane(kv ? 1u : 0u);  // lane 0 reads 0
            const bool head = kv && !(pkv && pkey == key);
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
                    rec_sh[wv][r] = key & a.shard_mask;
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

// Query: each processed k-mer loads its 256-bit shard (the lanes of a run
// load the same line, which one wave load serves once) and tests its masks;
// the step's answer ballot (E bits) is appended to a running 64-bit word so
// each store is one whole, aligned answer word.
template <int HC>
__global__ __launch_bounds__(256) void slide_query_kernel(SeqArgs a, Params P)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t E = slide_yield(P);
    const uint64_t ntasks = (a.nk + kSlideTask - 1) / kSlideTask;
    const uint64_t wstride = (uint64_t)gridDim.x * 4u;
    for (uint64_t task = (uint64_t)blockIdx.x * 4u + wv; task < ntasks; task += wstride) {
        const uint64_t t0 = task * kSlideTask;
        const uint64_t t1 = t0 + kSlideTask < a.nk ? t0 + kSlideTask : a.nk;
        uint64_t acc = 0;         // answers not yet stored, first at bit 0
        uint32_t nb = 0;          // how many (< 64)
        uint64_t word = t0 >> 6;  // answer word they belong to
        const SlideTask T(a, P, t0, lane);
        SlideWords D = slide_load(T, t0, lane);
        for (uint64_t base = t0; base < t1; base += E) {
            const SlideWords cur = D;
            D = slide_load(T, base + E, lane);  // the next step's words (past the task: unused)
            uint32_t key;
            uint64_t mk[4];
            bool pres = slide_step<HC>(P, T, cur, base, t1, lane, E, key, mk);
            if (pres) {
                uint64_t w[4];
                load_shard(a.filter, key & a.shard_mask, w);
                pres = ((~w[0] & mk[0]) | (~w[1] & mk[1]) | (~w[2] & mk[2]) | (~w[3] & mk[3])) == 0;
            }
            const uint64_t bits = __ballot(pres);  // bits 0 .. E-1
            acc |= bits << nb;
            const uint64_t spill = nb ? bits >> (64u - nb) : 0ull;
            nb += E;
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

// Kernel of a run-time family for this H: compile-time H for 1 .. 16,
// run-time above.
#define SBF_SLIDE_KERNEL(NAME, ARGS)                                                            \
    static void (*NAME##_for(uint32_t H))(ARGS, Params)                                         \
    {                                                                                           \
        switch (H) {                                                                            \
        case 1: return NAME<1>;   case 2: return NAME<2>;   case 3: return NAME<3>;             \
        case 4: return NAME<4>;   case 5: return NAME<5>;   case 6: return NAME<6>;             \
        case 7: return NAME<7>;   case 8: return NAME<8>;   case 9: return NAME<9>;             \
        case 10: return NAME<10>; case 11: return NAME<11>; case 12: return NAME<12>;           \
        case 13: return NAME<13>; case 14: return NAME<14>; case 15: return NAME<15>;           \
        case 16: return NAME<16>; default: return NAME<0>;                                     \
        }                                                                                       \
    }
SBF_SLIDE_KERNEL(slide_insert_kernel, SeqArgs)
SBF_SLIDE_KERNEL(slide_query_kernel, SeqArgs)
SBF_SLIDE_KERNEL(sbf_probe_rt_kernel, ProbeArgs)
#undef SBF_SLIDE_KERNEL

static uint32_t slide_blocks(uint64_t nk)
{
    const uint64_t tasks = (nk + kSlideTask - 1) / kSlideTask;
    uint64_t b = (tasks + 3) / 4;
    if (b > 16384)
        b = 16384;
    return (uint32_t)(b ? b : 1);
}

static uint32_t grid_for(uint64_t n)
{
    uint64_t b = (n + 255) / 256;
    if (b > 65536)
        b = 65536;
    return (uint32_t)(b ? b : 1);
}

// The Super Bloom filter takes the sliding kernels; the blocked Bloom
// comparator and the wide-block variant the per-k-mer ones.
static hipError_t gen_insert(const SeqArgs& a, const Params& P)
{
    if (P.kind == 0)
        hipLaunchKernelGGL(slide_insert_kernel_for(P.H), dim3(slide_blocks(a.nk)), dim3(256), 0, a.stream, a, P);
    else
        hipLaunchKernelGGL(generic_insert_kernel, dim3(grid_for(a.nk)), dim3(256), 0, a.stream, a, P);
    return hipGetLastError();
}

static hipError_t gen_query(const SeqArgs& a, const Params& P)
{
    if (P.kind == 0)
        hipLaunchKernelGGL(slide_query_kernel_for(P.H), dim3(slide_blocks(a.nk)), dim3(256), 0, a.stream, a, P);
    else
        hipLaunchKernelGGL(generic_query_kernel, dim3(grid_for((a.nk + 63) & ~63ull)), dim3(256), 0, a.stream, a,
                           P);
    return hipGetLastError();
}

static hipError_t gen_probe(const ProbeArgs& a, const Params& P)
{
    if (a.n == 0)
        return hipSuccess;
    uint64_t b = (a.n + 255) / 256;
    if (b > 8192)
        b = 8192;
    if (P.kind == 0)
        hipLaunchKernelGGL(sbf_probe_rt_kernel_for(P.H), dim3((uint32_t)b), dim3(256), 0, a.stream, a, P);
    else
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
