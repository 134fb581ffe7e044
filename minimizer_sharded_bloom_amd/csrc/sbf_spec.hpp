// sbf_spec.hpp -- compile-time specialized gfx950 kernels of the Super Bloom
// filter ([cuSBF] §IV-C..E, §IV-G "compile-time specialization").
//
// Work layout.  A 256-thread workgroup is four independent wave64s; each wave
// owns KPW = 63 * KL consecutive k-mer starts and a private slice of LDS.
//  - Lane l < 63 owns the KL consecutive k-mers starting at
//    p0 = wave_start + KL * l; lane 63 only computes hashes for lane 62's halo.
//  - Every lane loads its packed bases (KL/16 + 2 words, coalesced across the
//    wave), or decodes them from ASCII, and computes the m-mer hash and the
//    s-mer hash of its own KL positions exactly once; the w-1 m-mer hashes
//    and k-s s-mer hashes past its range come from lane l+1 through a lane
//    shift.
//  - The per-read query (sbf_query_reads_kernel) instead gives each lane 32
//    k-mers of one read of a batch and lets it hash the positions past them
//    itself, since lane l+1 may hold another read.
//  - Minimizer: a sliding-window minimum over the w m-mer hashes (van Herk /
//    Gil-Werman block prefix and suffix minima, block = w).
//  - Runs: consecutive valid k-mers of a lane with one shard ([cuSBF] §IV-D,
//    Fig. 3).  A wave scan numbers them; a run that continues the previous
//    lane's last run shares that lane's slot, so a super-k-mer cut by a lane
//    boundary still costs one record.
//  - Findere masks: R_i, the OR of the sector masks of the k-s+1 s-mers of
//    k-mer i, is built by binary doubling in a stream: each s-mer's masks and
//    each doubling level are computed once, at the step they first appear.
//  - Insert: run i's OR of R over its k-mers goes to an LDS record (shard,
//    four 64-bit words); then four adjacent lanes OR the four words of one
//    record into the filter in one instruction, which the memory system merges
//    into one request.
//  - Query: every run's shard is gathered into LDS by the whole wave at once
//    (two lanes per 32-byte shard); then k-mer i is present iff
//    (R_i & ~shard) == 0 over the used words ([cuSBF] Algorithm 2, Contains).
#pragma once

#include <type_traits>

#include "sbf_device.hpp"
#include "sbf_internal.hpp"

namespace sbf {

// KL_ = 0: 16 k-mers per lane, or 32 when the halo exceeds 16; a nonzero
// KL_ (16 or 32) fixes it.  A_ is the input: SBF_ALPHABET_DNA reads packed
// 2-bit codes and validity bits; SBF_ALPHABET_PROTEIN (5-bit letters) and
// SBF_ALPHABET_TRIPLET (6-bit codons of three bases) read the ASCII text and
// pack each lane's symbols in registers ([cuSBF] §IV-A); kDnaText reads DNA
// as ASCII and packs it in registers the same way, so an insert or query of
// a device sequence needs no separate packing pass.  kDnaReads is the per-read query
// of a batch of equal-length DNA reads: a lane takes 32 k-mer starts of one
// read and reads all 62 bases they span itself (no halo from lane l+1).
constexpr int kDnaText = 3;
constexpr int kDnaReads = 4;

template <int K_, int M_, int S_, int H_, int KL_ = 0, int A_ = 0>
struct Cfg {
    static constexpr int k = K_, m = M_, s = S_, H = H_, A = A_;
    static constexpr bool BASES = A_ == 0 || A_ == kDnaText || A_ == kDnaReads;  // 2-bit bases, 16 per word
    static constexpr bool OWN_HALO = A_ == kDnaReads;  // the lane hashes the positions past its own
    static constexpr int B = BASES ? 2 : (A_ == 1 ? 5 : 6);  // bits per symbol
    static constexpr int W = k - m + 1;    // m-mers per k-mer
    static constexpr int Z = k - s + 1;    // s-mers per k-mer (Findere z+1)
    static constexpr int HALO = (W - 1 > Z - 1) ? W - 1 : Z - 1;
    static constexpr int KL = KL_ ? KL_ : (HALO <= 16 ? 16 : 32);  // k-mers per lane
    static_assert(KL == 16 || KL == 32, "16 or 32 k-mers per lane");
    static_assert(HALO <= KL, "halo must come from the next lane alone");
    static_assert(BASES || KL == 16, "protein and triplet text: 16 symbols per lane");
    // DNA text at 32 k-mers per lane takes lane l+1's bases by DPP, and its
    // s-mers end within them; at 16 a lane loads its 48 bases itself
    static_assert(A_ != kDnaReads || KL == 32, "DNA reads: 32 k-mers per lane, 64 bases in four stream words");
    static constexpr int LW = 63;                    // working lanes per wave
    static constexpr int KPW = KL * LW;              // k-mers per wave
    // stream words per lane: for DNA KL/16 own code words and two of halo
    // (per-read query: its 64 bases and a zero word, which the 32-bit window
    // of its last m-mer may reach); for text, enough for every window of the
    // own positions plus one word
    static constexpr int ND = A_ == kDnaReads ? 5 : BASES ? KL / 16 + 2 : ((KL + (m > s ? m : s) - 1) * B + 31) / 32 + 1;
    static constexpr int NS = H < 4 ? H : 4;         // sectors in use
    static constexpr int NM = KL + W - 1;            // m-mer hashes per lane
    static constexpr int NZ = KL + Z - 1;            // s-mer hashes per lane
    static_assert(1 <= m && m <= k && k * B <= 64 && 1 <= s && s <= k && H >= 1, "bad parameters");
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// Window of N symbols of B bits starting at symbol j of a packed KK-mer x.
template <int KK, int N, int B = 2>
__device__ __forceinline__ uint64_t sub_bases(uint64_t x, int j)
{
    if constexpr (N * B >= 64)
        return x;
    else
        return (x >> (B * (KK - N - j))) & ((1ull << (B * N)) - 1ull);
}

// 32 bits of the lane's packed base stream starting at bit OFF (OFF compile
// time; the stream is D[0], D[1], ... with the first base in the top bits).
template <int OFF, int NDW>
__device__ __forceinline__ uint32_t stream_bits32(const uint32_t (&D)[NDW])
{
    constexpr int a = OFF >> 5, r = OFF & 31;
    static_assert(a + (r != 0) < NDW, "window past the lane's stream words");
    if constexpr (r == 0)
        return D[a];
    else
        return __builtin_amdgcn_alignbit(D[a], D[a + 1], 32 - r);
}

// Value of the N symbols of B bits starting at the lane's symbol P, first
// symbol most significant (N * B <= 64): one or two funnel shifts and a shift.
template <int P, int N, int B, int NDW>
__device__ __forceinline__ uint64_t bases_at(const uint32_t (&D)[NDW])
{
    constexpr int OFF = P * B, LEN = N * B;
    if constexpr (LEN <= 32) {
        const uint32_t w = stream_bits32<OFF>(D);
        return LEN == 32 ? (uint64_t)w : (uint64_t)(w >> (32 - LEN));
    } else {
        const uint32_t lo = stream_bits32<OFF + LEN - 32>(D);
        const uint32_t hi = LEN == 64 ? stream_bits32<OFF>(D) : stream_bits32<OFF>(D) >> (64 - LEN);
        return ((uint64_t)hi << 32) | lo;
    }
}

// Answer words are written in KL-bit pieces; the grid covers nk rounded up
// to 64 so every piece of every output word is written.
__host__ __device__ inline uint64_t round64(uint64_t x) { return (x + 63) & ~63ull; }

template <class C>
struct LaneCtx {
    uint64_t wstart;  // first k-mer of this wave (wave-uniform)
    uint64_t p0;      // first k-mer of this lane
    uint32_t lane;
    bool live;        // wave has work
};

template <class C>
__device__ __forceinline__ LaneCtx<C> lane_ctx(uint64_t nk_pad)
{
    LaneCtx<C> c;
    c.lane = threadIdx.x & 63u;
    const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x >> 6) + wib;
    c.wstart = wave * (uint64_t)C::KPW;
    c.live = c.wstart < nk_pad;
    c.p0 = c.wstart + (uint64_t)C::KL * c.lane;
    return c;
}

// Packed code words of the lane: KL/16 own words and two more for the halo
// (0 past the end of the sequence).  KPW is a multiple of 16, so the wave's
// first k-mer starts a code word.
template <class C>
__device__ __forceinline__ void load_codes(const SeqArgs& a, const LaneCtx<C>& c, uint32_t (&D)[C::ND])
{
    static_assert(C::KPW % 16 == 0, "wave start must align to a code word");
    const auto rs = word_buffer(a.codes, a.ncw, c.wstart >> 4);
    const uint32_t o = c.lane * (uint32_t)(C::KL / 16) * 4u;
#pragma unroll
    for (int j = 0; j < C::ND; ++j)
        D[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(o + 4u * j), 0, 0);
}

// x * 2 + (this lane's bit of the lane mask m): one v_addc with m as the
// carry-in, so a per-k-mer compare becomes a bit of a per-lane word in one
// instruction after the compare.
__device__ __forceinline__ uint32_t shift_in(uint32_t x, uint64_t m)
{
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(x), "s"(m));
    return r;
}

// Shard keys of the lane's KL k-mers: the low 32 bits of the minimizer hash
// (one m-mer hash per own position, halo from lane+1, van Herk sliding
// minimum with block size W).  The shard is key & shard_mask, applied where a
// shard is addressed; runs compare keys, which can only split a run where two
// minimizers share a shard -- the union and the answers are the same.
template <class C>
__device__ __forceinline__ void lane_shards(const uint32_t (&D)[C::ND], uint32_t (&shard)[C::KL])
{
    constexpr int W = C::W, KL = C::KL, NM = C::NM;
    uint64_t hm[NM];
    static_for<0, KL>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        hm[i] = hash_min(bases_at<i, C::m, C::B>(D));
        if constexpr (i < W - 1) {
            if constexpr (C::OWN_HALO)
                hm[KL + i] = hash_min(bases_at<KL + i, C::m, C::B>(D));
            else
                hm[KL + i] = from_next_lane(hm[i]);  // lane l+1's position i is this lane's KL+i
        }
    });
    if constexpr (W == 1) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
            shard[i] = (uint32_t)hm[i];
    } else {
        // Window [i, i+W) = tail of block i/W (suffix minimum at i) plus head of
        // block i/W+1 (prefix minimum at i+W-1); blocks are [bW, bW+W).
        // Pass 1 (descending) keeps the suffix minima of positions < KL in suf[]
        // and leaves hm[] untouched; pass 2 (ascending) carries the prefix
        // minimum in one register and closes window i = e-W+1 at each e.
        uint64_t suf[KL];
        uint64_t run = ~0ull;
#pragma unroll
        for (int j = NM - 1; j >= 0; --j) {
            const bool block_end = ((j % W) == W - 1) || (j == NM - 1);
            run = block_end ? hm[j] : (hm[j] < run ? hm[j] : run);
            if (j < KL)
                suf[j] = run;
        }
        uint64_t pre = ~0ull;
#pragma unroll
        for (int e = 0; e < NM; ++e) {
            pre = (e % W == 0) ? hm[e] : (hm[e] < pre ? hm[e] : pre);
            const int i = e - W + 1;
            if (i >= 0 && i < KL) {
                uint64_t mn;
                if (i % W == 0)
                    mn = suf[i];
                else
                    mn = suf[i] < pre ? suf[i] : pre;
                shard[i] = (uint32_t)mn;
            }
        }
    }
}

// Bit i set iff bits i .. i+KK-1 of v are all set: the zero bits of v are
// smeared down by KK-1 places (binary doubling), then complemented.  Bits
// within KK-1 of the top are not meaningful.
template <int KK>
__device__ __forceinline__ uint64_t valid_starts(uint64_t v)
{
    uint64_t z = ~v;
    static_for<0, 6>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int covered = 1 << j;  // z bit i covers offsets [0, covered) before this step
        if constexpr (covered < KK) {
            constexpr int sh = covered < KK - covered ? covered : KK - covered;
            z |= z >> sh;
        }
    });
    return ~z;
}

// Valid-k-mer bits of the lane (bit i: k-mer p0+i is valid and < nk), from
// the 64 validity bits starting at base p0 (three words, funnel shifts).
template <class C>
__device__ __forceinline__ uint32_t lane_valid(const SeqArgs& a, const LaneCtx<C>& c)
{
    static_assert(C::KL + C::k - 1 <= 64, "validity window");
    const auto rv = word_buffer(a.valid, a.nvw, c.wstart >> 5);
    const uint32_t bit = (uint32_t)(c.wstart & 31u) + (uint32_t)C::KL * c.lane;
    const uint32_t o = (bit >> 5) * 4u, off = bit & 31u;
    const uint32_t v0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rv, (int)o, 0, 0);
    const uint32_t v1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rv, (int)(o + 4u), 0, 0);
    const uint32_t v2 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rv, (int)(o + 8u), 0, 0);
    const uint64_t win = ((uint64_t)__builtin_amdgcn_alignbit(v2, v1, off) << 32) | __builtin_amdgcn_alignbit(v1, v0, off);
    const uint32_t v = (uint32_t)valid_starts<C::k>(win);
    const uint64_t rem = a.nk > c.p0 ? a.nk - c.p0 : 0;
    uint32_t keep = rem >= (uint64_t)C::KL ? (C::KL == 32 ? 0xFFFFFFFFu : (1u << C::KL) - 1u) : (1u << rem) - 1u;
    if (c.lane >= (uint32_t)C::LW)
        keep = 0;
    return v & keep;
}

// Validity bits of a protein dword (four letters, first in the low byte):
// byte j is valid iff it is an ASCII letter, i.e. c | 0x20 lies in 'a'..'z'.
// Setting bit 7 of every byte before subtracting keeps the bytes from
// borrowing from each other; bit j of the result is byte j.
__device__ __forceinline__ uint32_t letter_valid4(uint32_t w)
{
    const uint32_t xh = w | 0xA0A0A0A0u;        // lower case, bit 7 set
    const uint32_t ge = xh - 0x61616161u;       // bit 7: byte >= 'a'
    const uint32_t gt = xh - 0x7B7B7B7Bu;       // bit 7: byte > 'z'
    const uint32_t f = __builtin_amdgcn_bitop3_b32(ge, gt, w, 0x10) & 0x80808080u;  // ge & ~gt & ~w (ASCII)
    return (((f >> 7) * 0x00204081u) >> 21) & 0xFu;  // bits 7, 15, 23, 31 -> 0..3
}

// 32 DNA bases in eight dwords of ASCII (first base in the low byte of q[0])
// -> two stream words, first base most significant, and the returned
// validity bits (bit j: base j).  Per dword: the 2-bit codes c, as in the
// packing pass ((b >> 1) ^ (b >> 2)) & 3, gathered by one multiply into the
// top byte, first base most significant; and the invalid bytes at bit 7: a
// byte is valid iff, with bits 5 (case) and 7 cleared, it equals the letter
// of its code, and bit 7 is clear.  d7 has bits 5 and 7 of every byte clear,
// so d7 + 0x7F per byte sets bit 7 exactly for a nonzero byte and never
// carries.
__device__ __forceinline__ void dna_dword(uint32_t w, uint32_t& P, uint32_t& Zi)
{
    const uint32_t cc = __builtin_amdgcn_bitop3_b32(w >> 1, w >> 2, 0x03030303u, 0x28);  // (x ^ y) & m
    P = cc * 0x40100401u;  // code of byte j at bits 31-2j .. 30-2j
    const uint32_t e = __builtin_amdgcn_perm(0x74676361u, 0x74676361u, cc);  // "acgt" by code
    const uint32_t d7 = __builtin_amdgcn_bitop3_b32(w, 0xA0A0A0A0u, e, 0x12);     // ~k & (w ^ e)
    Zi = __builtin_amdgcn_bitop3_b32(d7 + 0x7F7F7F7Fu, w, 0x80808080u, 0xA8);     // (x | w) & m
}

__device__ __forceinline__ uint32_t decode_dna32(const uint32_t* q, uint32_t& S0, uint32_t& S1)
{
    uint32_t P[8], Zi[8];
#pragma unroll
    for (int d = 0; d < 8; ++d)
        dna_dword(q[d], P[d], Zi[d]);
    // code words: the top bytes of four products each
    S0 = __builtin_amdgcn_perm(P[0], P[1], 0x07030C0Cu) | __builtin_amdgcn_perm(P[2], P[3], 0x0C0C0703u);
    S1 = __builtin_amdgcn_perm(P[4], P[5], 0x07030C0Cu) | __builtin_amdgcn_perm(P[6], P[7], 0x0C0C0703u);
    // invalid flags of two dwords (bits 3,11,19,27 and 7,15,23,31) times
    // 1 + 2^7 + 2^14 + 2^21 land in bits 24..31 in base order, every
    // other partial product below bit 24 and on a bit of its own
    uint32_t V[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        V[g] = ((Zi[2 * g] >> 4) | Zi[2 * g + 1]) * 0x00204081u;
    return ~(__builtin_amdgcn_perm(V[1], V[0], 0x0C0C0703u) | __builtin_amdgcn_perm(V[3], V[2], 0x07030C0Cu));
}

// 16 DNA bases in four dwords of ASCII -> one stream word and 16 validity
// bits, as half of decode_dna32.
__device__ __forceinline__ uint32_t decode_dna16(const uint32_t* q, uint32_t& S0)
{
    uint32_t P[4], Zi[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        dna_dword(q[d], P[d], Zi[d]);
    S0 = __builtin_amdgcn_perm(P[0], P[1], 0x07030C0Cu) | __builtin_amdgcn_perm(P[2], P[3], 0x0C0C0703u);
    const uint32_t V0 = ((Zi[0] >> 4) | Zi[1]) * 0x00204081u;
    const uint32_t V1 = ((Zi[2] >> 4) | Zi[3]) * 0x00204081u;
    return ~__builtin_amdgcn_perm(V1, V0, 0x0C0C0703u) & 0xFFFFu;
}

// DNA text at 16 k-mers per lane: the lane loads the 48 bytes from its first
// base (three aligned 16-byte loads; neighbouring lanes' loads overlap and
// meet in the caches) and decodes them into its three stream words: its 16
// bases and the 32 that its k-mers reach past them.  Returns the lane's
// valid-k-mer bits, as lane_valid does for packed input.
template <class C>
__device__ __forceinline__ uint32_t load_dna_text16(const SeqArgs& a, const LaneCtx<C>& c, uint32_t (&D)[C::ND])
{
    static_assert(C::KL == 16 && C::ND == 3 && C::KL + C::k - 1 <= 48, "16 k-mers, 48 bases per lane");
    const uint64_t tb = a.nsym;
    const uint64_t b0 = c.wstart;  // a multiple of 16 (KPW = 1008)
    const uint64_t avail = tb > b0 ? tb - b0 : 0;
    const uint32_t nrec = avail < 0xFFFFFFFFull ? (uint32_t)avail : 0xFFFFFFFFu;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.text + (b0 < tb ? b0 : tb)), (short)0,
                                                      (int)nrec, 0x00020000);
    const uint32_t off = 16u * c.lane;
    uint32_t q[12];
    if (avail >= 63ull * 16 + 48) {
        // every byte of the wave lies before the end
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16u * j), 0, 0);
            q[4 * j] = v.x;
            q[4 * j + 1] = v.y;
            q[4 * j + 2] = v.z;
            q[4 * j + 3] = v.w;
        }
    } else {
        // the wave that reaches the end: byte loads, 0 past the last base
#pragma unroll
        for (int j = 0; j < 12; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)(off + 4u * j + b), 0, 0) << (8 * b);
            q[j] = w;
        }
    }
    const uint32_t v0 = decode_dna32(q, D[0], D[1]);
    const uint32_t v1 = decode_dna16(q + 8, D[2]);
    const uint32_t v = (uint32_t)valid_starts<C::k>(v0 | ((uint64_t)v1 << 32));
    const uint64_t rem = a.nk > c.p0 ? a.nk - c.p0 : 0;
    uint32_t keep = rem >= 16u ? 0xFFFFu : (1u << rem) - 1u;
    if (c.lane >= (uint32_t)C::LW)
        keep = 0;
    return v & keep;
}

// Text front end (protein and triplet filters, and DNA text): the lane's KL
// symbols (16 letters or codons, or 32 bases) are read from the ASCII text
// and packed in registers, first symbol most significant, B bits each, as
// D[0 ..]; the symbols past them come from lane l+1's packed words by DPP,
// and so do its validity bits.  A protein letter codes as (c - 1) & 31, its
// place in A..Z in either case; a base codes and validates as in the packing
// pass; a codon is its three bases' 2-bit codes, first base most significant,
// so the lane's 48 bases packed at 2 bits are its 16 codons at 6 bits.
// Returns the valid-k-mer bits of the lane (bit i: k-mer p0+i is valid and
// < nk).
template <class C>
__device__ __forceinline__ uint32_t load_text(const SeqArgs& a, const LaneCtx<C>& c, uint32_t (&D)[C::ND])
{
    constexpr int SB = C::A == 2 ? 3 : 1;  // bytes per symbol
    constexpr int NB = C::KL * SB;         // bytes per lane
    constexpr int NQ = NB / 16;            // 16-byte loads per lane
    constexpr int OB = C::KL * C::B;       // own stream bits
    constexpr int OW = OB / 32, OR = OB % 32;
    const uint64_t tb = a.nsym * (uint64_t)SB;  // bytes of whole symbols
    const uint64_t b0 = c.wstart * (uint64_t)SB;
    const uint64_t avail = tb > b0 ? tb - b0 : 0;
    const uint32_t nrec = avail < 0xFFFFFFFFull ? (uint32_t)avail : 0xFFFFFFFFu;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.text + (b0 < tb ? b0 : tb)), (short)0,
                                                      (int)nrec, 0x00020000);
    const uint32_t off = c.lane * (uint32_t)NB;
    uint32_t q[4 * NQ];
    if (avail >= 64ull * NB) {
        // every byte of the wave lies before the end
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16u * j), 0, 0);
            q[4 * j] = v.x;
            q[4 * j + 1] = v.y;
            q[4 * j + 2] = v.z;
            q[4 * j + 3] = v.w;
        }
    } else {
        // the wave that reaches the end: byte loads, 0 past the last symbol
#pragma unroll
        for (int j = 0; j < 4 * NQ; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)(off + 4u * j + b), 0, 0) << (8 * b);
            q[j] = w;
        }
    }
    uint32_t S[OW + (OR ? 1 : 0)];
    uint32_t own_valid = 0;
    if constexpr (C::A == 1) {
#pragma unroll
        for (int i = 0; i < OW + (OR ? 1 : 0); ++i)
            S[i] = 0;
#pragma unroll
        for (int t = 0; t < 4 * NQ; ++t) {
            const uint32_t codes = ((q[t] | 0x80808080u) - 0x01010101u) & 0x1F1F1F1Fu;  // (c - 1) & 31 per byte
            own_valid |= letter_valid4(q[t]) << (4 * t);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int P = 5 * (4 * t + jj), wd = P >> 5, r = P & 31;
                const uint32_t code = __builtin_amdgcn_ubfe(codes, 8 * jj, 5);
                if (r + 5 <= 32) {
                    S[wd] |= code << (27 - r);
                } else {
                    S[wd] |= code >> (r + 5 - 32);
                    S[wd + 1] |= code << (59 - r);
                }
            }
        }
    } else if constexpr (C::A == kDnaText) {
        static_assert(NQ == 2 && OW == 2 && OR == 0, "32 bases per lane");
        own_valid = decode_dna32(q, S[0], S[1]);
    } else {
        uint32_t cb[4 * NQ], nb[4 * NQ];
#pragma unroll
        for (int d = 0; d < 4 * NQ; ++d)
            encode_dword(q[d], cb[d], nb[d]);
#pragma unroll
        for (int u = 0; u < OW; ++u)
            S[u] = (cb[4 * u] << 24) | (cb[4 * u + 1] << 16) | (cb[4 * u + 2] << 8) | cb[4 * u + 3];
        // codon validity: four codons per three dwords (twelve bases); the
        // AND of bits 3c .. 3c+2 lands at bit 3c, then bits 0,3,6,9 -> 0..3
#pragma unroll
        for (int g = 0; g < 4 * NQ / 3; ++g) {
            const uint32_t v = nb[3 * g] | (nb[3 * g + 1] << 4) | (nb[3 * g + 2] << 8);
            uint32_t y = v & (v >> 1) & (v >> 2) & 0x249u;
            y = (y | (y >> 2)) & 0xC3u;
            y = (y | (y >> 4)) & 0xFu;
            own_valid |= y << (4 * g);
        }
    }
    // halo: lane l+1's packed words spliced after the own OB bits
    constexpr int NSW = OW + (OR ? 1 : 0);  // own stream words
    uint32_t N[C::ND];
#pragma unroll
    for (int t = 0; t < C::ND; ++t)
        N[t] = 0;
#pragma unroll
    for (int t = 0; t < NSW; ++t)
        N[t] = from_next_lane(S[t]);
#pragma unroll
    for (int u = 0; u < OW; ++u)
        D[u] = S[u];
#pragma unroll
    for (int t = 0; t < C::ND - OW; ++t) {
        if constexpr (OR == 0)
            D[OW + t] = N[t];
        else if (t == 0)
            D[OW] = S[OW] | (N[0] >> OR);
        else
            D[OW + t] = __builtin_amdgcn_alignbit(N[t - 1], N[t], OR);
    }
    // validity of the own symbols and then lane l+1's
    uint64_t win;
    if constexpr (C::KL == 32) {
        static_assert(C::KL + C::k - 1 <= 64, "validity window");
        win = own_valid | ((uint64_t)from_next_lane(own_valid) << 32);
    } else {
        static_assert(C::KL + C::k - 1 <= 32, "validity window");
        win = (uint32_t)(own_valid | (from_next_lane(own_valid) << C::KL));
    }
    const uint32_t v = (uint32_t)valid_starts<C::k>(win);
    const uint64_t rem = a.nk > c.p0 ? a.nk - c.p0 : 0;
    uint32_t keep = rem >= (uint64_t)C::KL ? (C::KL == 32 ? 0xFFFFFFFFu : (1u << C::KL) - 1u) : (1u << rem) - 1u;
    if (c.lane >= (uint32_t)C::LW)
        keep = 0;
    return v & keep;
}

// Stream words and valid-k-mer bits of the lane, from packed DNA or text.
template <class C>
__device__ __forceinline__ uint32_t lane_input(const SeqArgs& a, const LaneCtx<C>& c, uint32_t (&D)[C::ND])
{
    if constexpr (C::A == 0) {
        load_codes<C>(a, c, D);
        return lane_valid<C>(a, c);
    } else if constexpr (C::A == kDnaText && C::KL == 16) {
        return load_dna_text16<C>(a, c, D);
    } else {
        return load_text<C>(a, c, D);
    }
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

// Ordering point between the unrolled steps of a pass: the packed bases pass
// through an empty asm, so no hash of a later step can be computed before it
// (which would keep every hash live at once).  The first N words (all by
// default) pass; a constant word left out stays a constant.
template <int N = 0, int NDW>
__device__ __forceinline__ void step_fence(uint32_t (&D)[NDW])
{
    constexpr int n = N > 0 && N < NDW ? N : NDW;
#pragma unroll
    for (int j = 0; j < n; ++j)
        asm volatile("" : "+v"(D[j])::"memory");
}

// s-mer hash of the lane's own position Q (Q < KL).
template <class C, int Q>
__device__ __forceinline__ uint64_t smer_hash_at(const uint32_t (&D)[C::ND])
{
    return hash_s(bases_at<Q, C::s, C::B>(D));
}

// Streaming Findere masks.  Level l entry e = OR of the sector masks of
// s-mers e .. e + 2^l - 1.  R_I, the OR over the Z = k-s+1 s-mers of k-mer I,
// is split at the top level T = floor(log2 Z) into two halves (levels T-1 at
// I and I + 2^(T-1)) plus one stored entry per lower set bit of Z, so the top
// level is never stored: step<I>() hashes the s-mers new at k-mer I (all of
// 0..Z-1 at I = 0, then I+Z-1), builds the new entries of levels 0..T-1 and
// returns R_I = T0 | T1.  The first Z-1 own hashes and the Z-1 halo hashes of
// lane l+1 are computed by init(), and so are the next NPRE own hashes (the
// query computes them while its shard gather is in flight); every other hash
// in the step that first needs it, so few hashes are live at once.
template <class C, int NPRE = 0>
struct FindereMasks {
    static constexpr int NZ = C::NZ, Z = C::Z, TOP = ilog2c(Z), NLV = TOP > 0 ? TOP : 1;
    static constexpr int NH = Z > 1 ? Z - 1 : 1;
    static constexpr int NP = NPRE < C::KL - (Z - 1) ? NPRE : C::KL - (Z - 1);  // own positions Z-1 .. Z-2+NP
    uint64_t L[NLV][NZ][4];
    uint64_t head[NH];  // own hashes of positions 0 .. Z-2
    uint64_t halo[NH];  // hashes of positions KL .. KL+Z-2 (lane l+1's head)
    uint64_t pre[NP > 0 ? NP : 1];

    __device__ __forceinline__ void init(const uint32_t (&D)[C::ND])
    {
        static_for<0, Z - 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            head[q] = smer_hash_at<C, q>(D);
        });
        static_for<0, NP>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            pre[q] = smer_hash_at<C, Z - 1 + q>(D);
        });
        static_for<0, Z - 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            if constexpr (C::OWN_HALO)
                halo[q] = smer_hash_at<C, C::KL + q>(D);
            else
                halo[q] = from_next_lane(head[q]);
        });
    }

    template <int Q>
    __device__ __forceinline__ uint64_t hash_of(const uint32_t (&D)[C::ND])
    {
        if constexpr (Q < Z - 1)
            return head[Q];
        else if constexpr (Q < Z - 1 + NP)
            return pre[Q - (Z - 1)];
        else if constexpr (Q < C::KL)
            return smer_hash_at<C, Q>(D);
        else
            return halo[Q - C::KL];
    }

    // The hashes computed so far pass through an empty asm: a volatile asm
    // after this call (the gather's wait) cannot be moved above them.
    __device__ __forceinline__ void pin()
    {
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            asm volatile("" : "+v"(head[j]));
            asm volatile("" : "+v"(halo[j]));
        }
#pragma unroll
        for (int j = 0; j < NP; ++j)
            asm volatile("" : "+v"(pre[j]));
    }

    template <int I>
    __device__ __forceinline__ void step(const uint32_t (&D)[C::ND], uint64_t (&T0)[4], uint64_t (&T1)[4])
    {
        constexpr int qn = I == 0 ? 0 : I + Z - 1;
        constexpr int qe = I + Z - 1;
        static_for<qn, qe + 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            smer_masks<C>(hash_of<q>(D), L[0][q]);
        });
        static_for<1, TOP>([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int span = 1 << l;
            constexpr int e0 = (qn - span + 1) < 0 ? 0 : (qn - span + 1);
            constexpr int e1 = qe - span + 1;
            static_for<e0, e1 + 1>([&](auto ec) {
                constexpr int e = decltype(ec)::value;
#pragma unroll
                for (int w = 0; w < C::NS; ++w)
                    L[l][e][w] = L[l - 1][e][w] | L[l - 1][e + span / 2][w];
            });
        });
#pragma unroll
        for (int w = 0; w < 4; ++w)
            T0[w] = T1[w] = 0;
        if constexpr (TOP == 0) {
#pragma unroll
            for (int w = 0; w < C::NS; ++w)
                T0[w] = L[0][I][w];
        } else {
            constexpr int half = 1 << (TOP - 1);
#pragma unroll
            for (int w = 0; w < C::NS; ++w) {
                T0[w] = L[TOP - 1][I][w];
                T1[w] = L[TOP - 1][I + half][w];
            }
            // lower set bits of Z: stored entries after the top block
            static_for<0, TOP>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr ((Z >> j) & 1) {
                    constexpr int off = (Z >> (j + 1)) << (j + 1);
#pragma unroll
                    for (int w = 0; w < C::NS; ++w)
                        T0[w] |= L[j][I + off][w];
                }
            });
        }
    }
};

// Lane mask of v == 0 from one 64-bit compare (left to itself the compiler
// ORs the halves and compares 32 bits, one more vector instruction).
__device__ __forceinline__ uint64_t lanes_zero64(uint64_t v)
{
    uint64_t m;
    asm("v_cmp_eq_u64_e64 %0, 0, %1" : "=s"(m) : "v"(v));
    return m;
}

// Lanes whose k-mer has every bit of R = T0 | T1 set in the shard words W:
// per word, (T0 | T1) & ~W is one 3-input bit operation per 32-bit half and
// one 64-bit compare with zero; the words' lane masks are ANDed on the scalar
// unit.
template <class C>
__device__ __forceinline__ uint64_t lanes_present(const uint64_t (&T0)[4], const uint64_t (&T1)[4], const uint64_t (&W)[4])
{
    uint64_t present = ~0ull;
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const uint32_t lo = __builtin_amdgcn_bitop3_b32((uint32_t)T0[q], (uint32_t)T1[q], (uint32_t)W[q], 0x54);
        const uint32_t hi = __builtin_amdgcn_bitop3_b32((uint32_t)(T0[q] >> 32), (uint32_t)(T1[q] >> 32),
                                                        (uint32_t)(W[q] >> 32), 0x54);
        present &= lanes_zero64(((uint64_t)hi << 32) | lo);
    }
    return present;
}

// Run accumulation: Wr = (Wr & keep) | T0 | T1 with keep = 0 at a run start,
// all ones otherwise.
template <class C>
__device__ __forceinline__ void accumulate_run(uint64_t (&Wr)[4], uint32_t keep, const uint64_t (&T0)[4], const uint64_t (&T1)[4])
{
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const uint64_t t = T0[q] | T1[q];
        const uint32_t lo = __builtin_amdgcn_bitop3_b32((uint32_t)Wr[q], keep, (uint32_t)t, 0xEA);
        const uint32_t hi = __builtin_amdgcn_bitop3_b32((uint32_t)(Wr[q] >> 32), keep, (uint32_t)(t >> 32), 0xEA);
        Wr[q] = ((uint64_t)hi << 32) | lo;
    }
}

// ---------------------------------------------------------------------------
// Wave-level helpers.  Each wave owns a private slice of LDS: NSLOT records
// of (shard index, four 64-bit words).
// ---------------------------------------------------------------------------
constexpr int kSlots = 256;  // insert: records per wave (more go straight to the filter)
constexpr int kWaves = 4;    // waves per 256-thread workgroup

// Query records per wave before the direct path.  A wave of 2016 k-mers
// (32 per lane) of random sequence holds 2/(w+1) segments per k-mer: about
// 239 at w = 16 (standard deviation about 8), 269 at w = 14; short reads add
// one gap record per read but cut the segments there (about 213 per wave for
// 150-base reads).  280 slots keep a workgroup at 40.5 KB, so four fit in a
// CU's 160 KB; w <= 14 takes 352 slots and three workgroups.  Waves of 1008
// k-mers (16 per lane: the query's choice for w <= 11) hold about 168 at
// w = 11 and 336 at w = 5: 256 slots, or 352 when w <= 7.
template <class C>
constexpr int query_slots() { return C::KL == 32 ? (C::W <= 14 ? 352 : 280) : (C::W <= 7 ? 352 : 256); }

// Insert records per wave and round (a wave with more runs takes several
// rounds): 256, or 352 when w <= 8, where a wave of 1008 k-mers holds 2/(w+1)
// runs per k-mer, 224 at w = 8 and 336 at w = 5.
template <class C>
constexpr int insert_slots() { return C::W <= 8 ? 352 : kSlots; }

// NSLOT + 1 records per wave of (shard index, four 64-bit words).  The query
// numbers its records from 1 (record 0 is unused).  The
// indices sit in their own array: pass A writes one per k-mer, and at a
// 4-byte stride neighbouring records fall in different LDS banks.
template <int NSLOT>
struct WaveLdsN {
    uint32_t idx[kWaves][NSLOT + 1];
    alignas(16) uint64_t words[kWaves][NSLOT + 1][4];  // 32-byte records, 16-byte halves
};

// Gather of a wave's records 1 .. total into LDS: record r is the RB-byte
// shard (idx[r] & shard_mask) of the filter, copied to words + RB * r.  Each
// load goes straight from the filter into LDS: one instruction fills a group
// of 64 * 16 / RB consecutive records (1 KiB, lane l at byte 16 l), so all
// groups' loads are in flight at once and no VGPR stages them.  A lane past
// the last record loads nothing.  idx holds NSLOT + 1 entries and words
// NSLOT + 1 records; total <= NSLOT.  The loads are complete when this
// returns.
template <int RB, int NSLOT, bool WAIT = true>
__device__ __forceinline__ void gather_records(const uint64_t* __restrict__ filter, uint32_t shard_mask,
                                               const uint32_t* idx, char* words, uint32_t total, uint32_t lane)
{
    constexpr int LPR = RB / 16;       // lanes per record
    constexpr int RPG = 64 / LPR;      // records per group
    constexpr int NG = (NSLOT + RPG - 1) / RPG;  // groups (the last may be partial)
    constexpr int CH = 8;                        // groups whose indices are read before their loads
    const uint32_t part = lane % LPR;
    const uint32_t r0 = 1u + lane / LPR;
#pragma unroll
    for (int g0 = 0; g0 < NG; g0 += CH) {
        if ((uint32_t)(RPG * g0) >= total)
            break;
        uint32_t sh[CH];
#pragma unroll
        for (int j = 0; j < CH && g0 + j < NG; ++j) {
            if ((uint32_t)(RPG * (g0 + j)) >= total)
                break;
            const uint32_t r = r0 + (uint32_t)(RPG * (g0 + j));
            sh[j] = idx[r <= total ? r : 0u] & shard_mask;
        }
#pragma unroll
        for (int j = 0; j < CH && g0 + j < NG; ++j) {
            if ((uint32_t)(RPG * (g0 + j)) >= total)
                break;
            if (r0 + (uint32_t)(RPG * (g0 + j)) <= total)
                __builtin_amdgcn_global_load_lds(filter + (uint64_t)(RB / 8) * sh[j] + 2u * part,
                                                 words + RB * (1 + RPG * (g0 + j)), 16, 0, 0);
        }
    }
    if constexpr (WAIT)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Inclusive prefix sum over the wave: DPP row shifts by 1, 2, 4 and 8 sum
// within each row of 16 lanes, then the row_bcast:15 and row_bcast:31 moves
// carry the totals of rows 0 and 0..1 into the later rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
    return x;
}


// Run starts of a lane: bit i set if k-mer i is valid and does not continue
// the previous one (invalid, or another shard).  Runs double as query
// segments.  The shard comparisons enter a bit word through shift_in, last
// k-mer first.
template <class C>
__device__ __forceinline__ uint32_t run_starts(uint32_t vk, const uint32_t (&shard)[C::KL])
{
    uint32_t ne = 0;  // bit i (i >= 1): shard i differs from shard i-1
#pragma unroll
    for (int i = C::KL - 1; i >= 1; --i)
        ne = shift_in(ne, __builtin_amdgcn_ballot_w64(shard[i] != shard[i - 1]));
    ne = (ne << 1) | 1u;
    return vk & (ne | ~(vk << 1));
}

// Does this lane's first run continue the previous lane's last run?  Then the
// two share one record slot (the previous lane's last).
template <class C>
__device__ __forceinline__ bool continues_previous(uint32_t vk, const uint32_t (&shard)[C::KL], uint32_t lane)
{
    const uint32_t prev_last_valid = from_prev_lane((vk >> (C::KL - 1)) & 1u);
    const uint32_t prev_last_shard = from_prev_lane(shard[C::KL - 1]);
    return lane > 0 && (vk & 1u) && prev_last_valid && shard[0] == prev_last_shard;
}

// Record numbers of a query lane's k-mers; returns the wave's record count.
// Records number, from 1 across the wave, the segments (runs of valid k-mers
// with one shard) and the gaps (runs of invalid k-mers); one that continues
// the previous lane's last keeps its number.  Every k-mer can then write its
// shard index into its own record with no branch and no validity test: a
// segment's k-mers all carry its shard, and a gap's record holds some index
// whose answers the validity bits clear.
// With GAPS false (the per-read query, whose lanes end in the invalid starts
// past their read's last k-mer) only a gap that opens a lane gets a record
// of its own, one that continues no other lane's; every other gap shares the
// record of the segment before it.  The k-mers must then write their records
// last k-mer first, so that the segment's own first k-mer writes last.
template <class C, bool GAPS = true>
__device__ __forceinline__ uint32_t query_records(uint32_t vk, const uint32_t (&shard)[C::KL], uint32_t lane,
                                                  uint32_t (&rec)[C::KL], uint32_t& gs_out, uint32_t& first_out)
{
    constexpr uint32_t all = C::KL == 32 ? 0xFFFFFFFFu : (1u << C::KL) - 1u;
    const uint32_t st = run_starts<C>(vk, shard);
    const uint32_t gs = GAPS ? (st | (~vk & ((vk << 1) | 1u))) & all  // plus gap starts
                             : st | (~vk & 1u);                       // plus a gap that opens the lane
    const uint32_t prev_valid = from_prev_lane((vk >> (C::KL - 1)) & 1u);
    const uint32_t prev_shard = from_prev_lane(shard[C::KL - 1]);
    const bool cont = lane > 0 && ((vk & 1u) ? (prev_valid && shard[0] == prev_shard) : (GAPS && !prev_valid));
    const uint32_t cin = cont ? 1u : 0u;
    const uint32_t n = __popc(gs) - cin;
    const uint32_t incl = wave_incl_scan(n);
    const uint32_t first = incl - n - cin;  // record of the lane's k-mers before its first start
#pragma unroll
    for (int i = 0; i < C::KL; ++i)
        rec[i] = __popc(gs & ((2u << i) - 1u)) + first;
    gs_out = gs;
    first_out = first;
    return __builtin_amdgcn_readlane(incl, 63);
}

// Gap records point at shard 0.  The k-mers of a gap wrote the keys of
// invalid windows to it; each of those would cost the gather a line from
// HBM, while shard 0 stays in L2 after its first load.  The answers of a gap
// are cleared by the validity bits whatever its record holds.  Runs after the
// k-mers' own writes (LDS writes of one wave land in program order).
template <class C>
__device__ __forceinline__ void point_gaps_at_shard0(uint32_t* idx, uint32_t vk, uint32_t gs, uint32_t first)
{
    constexpr uint32_t all = C::KL == 32 ? 0xFFFFFFFFu : (1u << C::KL) - 1u;
    const uint32_t g = ~vk & all;
    uint32_t gst = g & ~(g << 1);  // first k-mer of each gap piece in the lane
    while (gst) {
        const uint32_t b = (uint32_t)__builtin_ctz(gst);
        idx[__popc(gs & ((2u << b) - 1u)) + first] = 0u;
        gst &= gst - 1u;
    }
}

template <class C>
__device__ __forceinline__ void global_or_record(uint64_t* __restrict__ filter, uint32_t shard, const uint64_t (&Wm)[4])
{
    uint64_t* base = filter + 4ull * shard;
#pragma unroll
    for (int q = 0; q < C::NS; ++q)
        atomic_or_u64(base + q, Wm[q]);
}

// Insert ([cuSBF] Algorithm 1).  Pass A: shards, validity and run starts;
// a wave scan gives each run a record slot.  Pass B: each run's sector masks
// go to its slot (a run continuing the previous lane's last run ORs into that
// slot).  Flush: four adjacent lanes OR the four words of one record into the
// filter.  With dense minimizers a wave with more runs than slots does this
// in rounds of slots.
template <class C>
__global__ __launch_bounds__(256) void sbf_insert_kernel(SeqArgs a)
{
    constexpr int kInsSlots = insert_slots<C>();
    __shared__ WaveLdsN<kInsSlots> lds;
    const LaneCtx<C> c = lane_ctx<C>(a.nk);
    if (!c.live)
        return;  // whole wave
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar LDS bases
    uint32_t D[C::ND];
    const uint32_t vk = lane_input<C>(a, c, D);
    uint32_t shard[C::KL];
    lane_shards<C>(D, shard);

    // pass A: slots
    const uint32_t st = run_starts<C>(vk, shard);
    const uint32_t cin = continues_previous<C>(vk, shard, c.lane) ? 1u : 0u;
    const uint32_t nrec = __popc(st) - cin;
    const uint32_t incl = wave_incl_scan(nrec);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    const uint32_t base = incl - nrec;

    // Dense minimizers (w <= 8) go in rounds of kInsSlots records: a later
    // round repeats pass B and keeps the records of its own range, so every
    // record is flushed merged.  Elsewhere one round serves, and a record
    // past the slots (a rare wave) goes straight to the filter from its lane;
    // the rounds would keep pass B's inputs live across the loop, which
    // costs those kernels about 50 VGPRs.
    constexpr bool kRounds = C::W <= 8;
    const uint32_t nrounds = kRounds ? total : (total ? 1u : 0u);
    for (uint32_t r0 = 0; r0 < nrounds; r0 += (uint32_t)kInsSlots) {
        if (r0)
            wave_lds_sync();  // the previous round's flush has read its records
        // pass B: run masks -> records
        FindereMasks<C> fm;
        fm.init(D);
        uint64_t Wr[4] = {0, 0, 0, 0};
        uint64_t first[4] = {0, 0, 0, 0};
        const uint32_t slot0 = base - cin - r0;  // this lane's first own record in this round's slots
        static_for<0, C::KL>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            uint64_t T0[4], T1[4];
            fm.template step<i>(D, T0, T1);
            const bool vi = (vk >> i) & 1u;
            // a run start clears the run masks; an invalid k-mer may add to
            // them, as it never lies inside a run and the next start clears
            // them again
            const uint32_t keep = ((st >> i) & 1u) ? 0u : 0xFFFFFFFFu;
            accumulate_run<C>(Wr, keep, T0, T1);
            // the run ends here if the next k-mer does not continue it
            bool ends;
            if constexpr (i == C::KL - 1)
                ends = vi;
            else
                ends = vi && (((st >> (i + 1)) & 1u) || !((vk >> (i + 1)) & 1u));
            if (ends) {
                const uint32_t ridx = __popc(st & ((2u << i) - 1u)) - 1u;
                if (ridx == 0 && cin) {
#pragma unroll
                    for (int w = 0; w < C::NS; ++w)
                        first[w] = Wr[w];
                } else {
                    const uint32_t slot = slot0 + ridx;  // below kInsSlots iff in this round
                    if (slot < (uint32_t)kInsSlots) {
                        lds.idx[wv][slot] = shard[i];
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            lds.words[wv][slot][w] = Wr[w];
                    } else if constexpr (!kRounds) {
                        global_or_record<C>(a.filter, shard[i] & a.shard_mask, Wr);
                    }
                }
            }
            step_fence(D);
        });
        wave_lds_sync();
        // first runs continuing the previous lane: OR into its last record
        if (cin) {
            const uint32_t slot = base - 1u - r0;
            if (slot < (uint32_t)kInsSlots) {
#pragma unroll
                for (int w = 0; w < C::NS; ++w)
                    __hip_atomic_fetch_or(&lds.words[wv][slot][w], first[w], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WAVEFRONT);
            } else if constexpr (!kRounds) {
                global_or_record<C>(a.filter, shard[0] & a.shard_mask, first);
            }
        }
        wave_lds_sync();

        // flush: lane -> (record, word)
        const uint32_t left = total - r0;
        const uint32_t T = left < (uint32_t)kInsSlots ? left : (uint32_t)kInsSlots;
        for (uint32_t r = c.lane; r < 4u * T; r += 64u) {
            const uint32_t rec = r >> 2, q = r & 3u;
            if (q < (uint32_t)C::NS) {
                const uint64_t m = lds.words[wv][rec][q];
                if (m)
                    atomic_or_u64(a.filter + 4ull * (lds.idx[wv][rec] & a.shard_mask) + q, m);
            }
        }
    }
}

// Query of one lane's KL k-mers, each on its own: the k-mer from its base
// window, minimizer over its w m-mers, one shard load, all s-mer masks.  The
// path for waves whose runs exceed the LDS slots (very short runs); a runtime
// loop keeps it small.
// The k-mer starting at the lane's symbol i (a run-time index): the 64
// stream bits from bit i*B, cut to k symbols.
template <class C>
__device__ __forceinline__ uint64_t kmer_at_lane(const uint32_t (&D)[C::ND], int i)
{
    uint32_t d0, d1, d2, r;
    if constexpr (C::BASES) {
        const bool hi16 = i >= 16;
        d0 = hi16 ? D[1] : D[0];
        d1 = hi16 ? D[2] : D[1];
        d2 = hi16 ? D[C::ND > 3 ? 3 : C::ND - 1] : D[2];  // i >= 16 only when KL = 32 (ND >= 4)
        r = 2u * (uint32_t)(i & 15);
    } else {
        const uint32_t off = (uint32_t)i * C::B, wa = off >> 5;
        r = off & 31u;
        d0 = d1 = d2 = 0;
#pragma unroll
        for (int j = 0; j < C::ND; ++j) {
            if (wa == (uint32_t)j) {
                d0 = D[j];
                d1 = j + 1 < C::ND ? D[j + 1 < C::ND ? j + 1 : j] : 0u;
                d2 = j + 2 < C::ND ? D[j + 2 < C::ND ? j + 2 : j] : 0u;
            }
        }
    }
    const uint64_t win = ((uint64_t)funnel_hi(d0, d1, r) << 32) | funnel_hi(d1, d2, r);
    return C::k * C::B >= 64 ? win : win >> (64 - C::k * C::B);
}

template <class C>
__device__ __forceinline__ uint32_t query_lane_direct(const SeqArgs& a, const uint32_t (&D)[C::ND], uint32_t vk)
{
    uint32_t bits = 0;
    for (int i = 0; i < C::KL; ++i) {
        if (!((vk >> i) & 1u))
            continue;
        const uint64_t x = kmer_at_lane<C>(D, i);
        uint64_t mn = ~0ull;
#pragma unroll
        for (int j = 0; j < C::W; ++j) {
            const uint64_t h = hash_min(sub_bases<C::k, C::m, C::B>(x, j));
            mn = h < mn ? h : mn;
        }
        uint64_t w[4];
        load_shard(a.filter, (uint32_t)mn & a.shard_mask, w);
        uint64_t R[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            uint64_t mk[4];
            smer_masks<C>(hash_s(sub_bases<C::k, C::s, C::B>(x, j)), mk);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                R[q] |= mk[q];
        }
        uint32_t hit = 1u;
#pragma unroll
        for (int q = 0; q < C::NS; ++q)
            hit &= (uint32_t)((R[q] & w[q]) == R[q]);
        bits |= hit << i;
    }
    return bits;
}

// Query ([cuSBF] Algorithm 2) of one lane's KL k-mers, given its stream
// words D and valid-k-mer bits vk.  Pass A: shards and per k-mer the LDS
// record of its segment (a run of one shard) or gap (a run of invalid
// k-mers), numbered from 1 across the wave.  Every k-mer writes its shard
// index to its record: all k-mers of a segment carry the same shard, so no
// write needs a branch.  Gather: the wave loads every record's 32-byte shard
// into LDS at once, two lanes per shard.  Pass B (straight-line): k-mer i
// reads the words of its record and is present iff every bit of its Findere
// mask R_i is set: (R_i & W) == R_i; invalid k-mers answer 0.  Returns the
// answer bits (bit i: k-mer i).
// s-mer hashes of pass B that the query computes before waiting for its
// gather (each holds two VGPRs from then to its step).  Where w <= 16,
// k-s+1 <= 4 and H <= 4 (the operating point (31,16,28,4) among them) eight,
// or four where the lane also hashes its own halo, fit the kernels' 128
// VGPRs: 1.5 % off the query out of every cache, 0.5 % at 512 MiB.  Larger
// windows, more s-mers or more hashes would lose a wave per SIMD to them.
template <class C>
constexpr int kQueryPreHashes()
{
    return (C::W <= 16 && C::Z <= 4 && C::H <= 4) ? (C::OWN_HALO ? 4 : 8) : 0;
}

template <class C, bool GAPS, int NSLOT>
__device__ __forceinline__ uint32_t query_lane(const SeqArgs& a, uint32_t (&D)[C::ND], uint32_t vk,
                                               uint32_t lane, int wv, WaveLdsN<NSLOT>& lds)
{
    uint32_t total;
    uint32_t rec[C::KL];
    {
        uint32_t shard[C::KL];
        lane_shards<C>(D, shard);
        // pass A: segment and gap records, shard indices into LDS
        uint32_t gs, first;
        total = query_records<C, GAPS>(vk, shard, lane, rec, gs, first);
        if (total <= (uint32_t)NSLOT) {
            if constexpr (GAPS) {
#pragma unroll
                for (int i = 0; i < C::KL; ++i)
                    lds.idx[wv][rec[i]] = shard[i];
                point_gaps_at_shard0<C>(lds.idx[wv], vk, gs, first);
            } else {
                // last k-mer first: a segment's first k-mer writes its record last
#pragma unroll
                for (int i = C::KL - 1; i >= 0; --i)
                    lds.idx[wv][rec[i]] = shard[i];
            }
        }
    }
    uint32_t bits;
    if (total <= (uint32_t)NSLOT) {
        wave_lds_sync();
        gather_records<32, NSLOT, false>(a.filter, a.shard_mask, lds.idx[wv],
                                         reinterpret_cast<char*>(&lds.words[wv][0][0]), total, lane);
        __builtin_amdgcn_s_setprio(0);
        // the first s-mer hashes of pass B while the gather is in flight
        FindereMasks<C, kQueryPreHashes<C>()> fm;
        fm.init(D);
        fm.pin();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        wave_lds_sync();

        // pass B
        bits = 0;
        static_for<0, C::KL>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            uint64_t T0[4], T1[4];
            fm.template step<i>(D, T0, T1);
            const ulonglong2* ws = reinterpret_cast<const ulonglong2*>(lds.words[wv][rec[i]]);
            const ulonglong2 w01 = ws[0];
            uint64_t wq[4] = {w01.x, w01.y, 0, 0};
            if constexpr (C::NS > 2) {
                const ulonglong2 w23 = ws[1];
                wq[2] = w23.x;
                wq[3] = w23.y;
            }
            bits = shift_in(bits, lanes_present<C>(T0, T1, wq));  // k-mer i lands at bit KL-1-i
            step_fence<C::OWN_HALO ? 4 : 0>(D);  // the per-read query's zero word stays a constant
        });
        bits = (__builtin_bitreverse32(bits) >> (32 - C::KL)) & vk;
    } else {
        bits = query_lane_direct<C>(a, D, vk);
    }
    return bits;
}

// Query of a sequence: each lane answers KL consecutive k-mer starts.
template <class C>
__global__ __launch_bounds__(256) void sbf_query_kernel(SeqArgs a)
{
    constexpr int kQuerySlots = query_slots<C>();
    __shared__ WaveLdsN<kQuerySlots> lds;
    const uint64_t nk_pad = round64(a.nk);
    const LaneCtx<C> c = lane_ctx<C>(nk_pad);
    if (!c.live)
        return;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar LDS bases
    uint32_t D[C::ND];
    __builtin_amdgcn_s_setprio(1);  // pass A first: its gather is what the other waves wait on
    const uint32_t vk = lane_input<C>(a, c, D);
    const uint32_t bits = query_lane<C, true>(a, D, vk, c.lane, wv, lds);
    if (c.lane < (uint32_t)C::LW && c.p0 < nk_pad) {
        if constexpr (C::KL == 16)
            reinterpret_cast<uint16_t*>(a.out)[c.p0 >> 4] = (uint16_t)bits;
        else
            reinterpret_cast<uint32_t*>(a.out)[c.p0 >> 5] = bits;
    }
}

// Per-read query input.  Lane g of the launch (g = 64 * wave + lane) takes
// chunk c = g mod R of read r = g / R: the k-mer starts 32c .. 32c+31 of the
// read.  It loads the 64 bytes from base 32c of the read (the 62 its k-mers
// span, and two more) itself, as four stream words; nothing comes from lane
// l+1.  Reads start anywhere: the lane loads the 17 aligned dwords around its
// bytes and shifts them into place.  Returns the lane's valid-k-mer bits:
// k-mer 32c+i is valid iff its k bases are and it is one of the read's
// len - k + 1 k-mers.
template <class C>
__device__ __forceinline__ uint32_t reads_input(const SeqArgs& a, uint64_t g0, uint32_t lane, uint32_t (&D)[C::ND])
{
    static_assert(C::ND == 5, "64 bases per lane and a zero word");
    // the batch holds fewer than 2^32 chunks and stride <= 2^25 bytes, so a
    // wave's bytes lie within 65 strides of its first (host checks)
    const uint32_t R = a.rchunks;
    const uint32_t g = (uint32_t)g0 + lane;
    const uint32_t r = g / R, c = g - r * R;
    const uint32_t r0 = (uint32_t)g0 / R, c0 = (uint32_t)g0 - r0 * R;  // the wave's first chunk
    // byte addresses relative to the dword below the wave's first byte
    const uintptr_t first = reinterpret_cast<uintptr_t>(a.text) + (uint64_t)r0 * a.stride + 32u * c0;
    const char* base = reinterpret_cast<const char*>(first & ~(uintptr_t)3);
    const uint64_t end = reinterpret_cast<uintptr_t>(a.text) + a.nsym - reinterpret_cast<uintptr_t>(base);
    const uint32_t nrec = end < 0xFFFFFFFFull ? (uint32_t)end : 0xFFFFFFFFu;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)nrec, 0x00020000);
    const uint32_t lb = (uint32_t)(reinterpret_cast<uintptr_t>(a.text) + (uint64_t)r * a.stride + 32u * c -
                                   reinterpret_cast<uintptr_t>(base));
    const uint32_t o = lb & ~3u, sh = lb & 3u;
    uint32_t q[17];
    const bool whole = __builtin_amdgcn_ballot_w64(o + 68u > nrec) == 0;  // wave-uniform
    if (whole) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(o + 16u * j), 0, 0);
            q[4 * j] = v.x;
            q[4 * j + 1] = v.y;
            q[4 * j + 2] = v.z;
            q[4 * j + 3] = v.w;
        }
        q[16] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(o + 64u), 0, 0);
    } else {
        // a wave that reaches the end of the batch: byte loads, 0 past it
#pragma unroll
        for (int j = 0; j < 17; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)(o + 4u * j + b), 0, 0) << (8 * b);
            q[j] = w;
        }
    }
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        w[j] = __builtin_amdgcn_alignbyte(q[j + 1], q[j], sh);
    const uint32_t v0 = decode_dna32(w, D[0], D[1]);
    const uint32_t v1 = decode_dna32(w + 8, D[2], D[3]);
    D[4] = 0;
    const uint32_t v = (uint32_t)valid_starts<C::k>(v0 | ((uint64_t)v1 << 32));
    const uint32_t left = a.rlen - (uint32_t)C::k + 1u - 32u * c;  // the read's k-mers from 32c on
    uint32_t keep = left >= 32u ? 0xFFFFFFFFu : (1u << left) - 1u;
    if (g >= a.nk)
        keep = 0;
    return v & keep;
}

// Per-read query of a batch of equal-length reads (lanes as in reads_input).
// A lane's k-mers all lie in one read, so no lane spends work on the starts
// that straddle two reads; the answers of read r are 32-bit words R*r ..
// R*r + R-1, k-mer 32j + i at bit i of word j, 0 past the read's last k-mer.
template <class C>
__global__ __launch_bounds__(256) void sbf_query_reads_kernel(SeqArgs a)
{
    constexpr int kQuerySlots = query_slots<C>();
    __shared__ WaveLdsN<kQuerySlots> lds;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t g0 = ((uint64_t)blockIdx.x * 4u + (uint32_t)wv) * 64u;
    if (g0 >= a.nk)
        return;
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t D[C::ND];
    __builtin_amdgcn_s_setprio(1);  // pass A first: its gather is what the other waves wait on
    const uint32_t vk = reads_input<C>(a, g0, lane, D);
    const uint32_t bits = query_lane<C, false>(a, D, vk, lane, wv, lds);
    if (g0 + lane < a.nk)
        reinterpret_cast<uint32_t*>(a.out)[g0 + lane] = bits;
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
        // one k-mer with its own shard: test its Z*H bits one by one (a
        // shift each) rather than build and compare sector masks
        uint32_t hit = 1u;
#pragma unroll
        for (int j = 0; j < C::Z; ++j) {
            const uint64_t h = hash_s(sub_bases<C::k, C::s>(x, j));
#pragma unroll
            for (int t = 0; t < C::H; ++t)
                hit &= (uint32_t)(w[t & 3] >> bit_addr<C::H>(h, t));
        }
        cnt += hit & 1u;
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

// a.nk counts the batch's chunks (R per read), one lane each
template <class C>
hipError_t launch_query_reads(const SeqArgs& a, const Params&)
{
    const uint64_t blocks = (a.nk + 255) / 256;
    hipLaunchKernelGGL(sbf_query_reads_kernel<C>, dim3((uint32_t)blocks), dim3(256), 0, a.stream, a);
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

// The query takes 32 k-mers per lane while k-s+1 <= 8 and w >= 12: its
// per-lane work (code loads, halo moves, scan, gather) is then spread over
// twice the k-mers.  More s-mers per k-mer make the doubling levels too large
// for 32 (over 160 VGPRs); denser minimizers (w <= 11) would give a 2016-k-mer
// wave more segments than its LDS slots; and the insert measures faster at 16.
// At 32 k-mers per lane a query also reads the DNA as ASCII itself, so that a
// device sequence is packed in registers instead of by a pass of its own.
template <int K, int M, int S, int H>
KernelSet spec_set()
{
    using C = Cfg<K, M, S, H>;
    constexpr bool kQ32 = K - S + 1 <= 8 && K - M + 1 >= 12;
    using CQ = Cfg<K, M, S, H, (kQ32 ? 32 : 0)>;
    KernelSet ks;
    ks.insert = &launch_insert<C>;
    ks.insert_text = &launch_insert<Cfg<K, M, S, H, 0, kDnaText>>;
    ks.query = &launch_query<CQ>;
    if constexpr (kQ32) {
        ks.query_text = &launch_query<Cfg<K, M, S, H, 32, kDnaText>>;
        ks.query_reads = &launch_query_reads<Cfg<K, M, S, H, 32, kDnaReads>>;
    }
    ks.probe = &launch_probe<C>;
    ks.specialized = 1;
    return ks;
}

}  // namespace sbf
