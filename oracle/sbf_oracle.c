/*
 * sbf_oracle.c -- plain, single-threaded CPU oracle of the Super Bloom filter.
 *
 * TEST INFRASTRUCTURE ONLY (see sbf_oracle.h).  Slow on purpose: every k-mer
 * is packed, minimized, hashed and tested from scratch.
 *
 * Source: [cuSBF] = "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
 * Sequence Data on Modern GPUs" (Dortmann, Vieth, Schmidt).
 *
 * Readings fixed here where [cuSBF] leaves a step open:
 *  - Codes: A/a=0, C/c=1, G/g=2, T/t=3; any other byte is an invalid symbol
 *    ([cuSBF] §IV-A names the 2-bit DNA alphabet, not the code order).
 *  - A k-mer is packed with its first base in the most significant bits
 *    (shift-left-and-OR of [cuSBF] §IV-C / §IV-E); sub-window i is the
 *    window starting at base i of the k-mer.
 *  - h_min(v) = u ^ (u >> 32) with u = (v + G) * C1 mod 2^64: one
 *    multiplicative mix ([cuSBF] §IV-G, role-specialized hashing), folded so
 *    the low bits used for the shard depend on every base.
 *  - h_s(v) = mix(v + G), mix = the SplitMix64 finalizer (two multiplies and
 *    three xorshifts): the "stronger mix" of [cuSBF] §IV-G, SplitMix-style as
 *    the CPU reference of [cuSBF] §V-D.
 *    G  = 0x9E3779B97F4A7C15 (2^64 / golden ratio),
 *    C1 = 0xBF58476D1CE4E5B9, C2 = 0x94D049BB133111EB (SplitMix64).
 *  - Bit address: for H <= 10, slice t of width floor(64/H), its low 6 bits
 *    ([cuSBF] §IV-G bit-slicing); for H > 10, the top 6 bits of hs * salt_t
 *    with salt_t = mix((t+1) * G), the t-th SplitMix64 output of seed 0 (the
 *    golden-ratio-derived per-index salt of §IV-G).  A salt of the form
 *    (2t+1) * G would make the H addresses an arithmetic progression.
 *  - Shard count: the smallest power of two >= ceil(bits/256), at least 1
 *    ([cuSBF] §IV-B).  Hash index t lives in word t mod 4 of the shard.
 *  - Wide variant (OSBF_KIND_WIDE), the layout [cuSBF] §V-D attributes to the
 *    CPU Super Bloom reference: 512-bit blocks, each hash index addressing any
 *    bit of the block.  Block count: the smallest power of two >=
 *    ceil(bits/512).  Address of hash t: for H <= 7, slice t of width
 *    floor(64/H), its low 9 bits; for H > 7, the top 9 bits of hs * salt_t
 *    (salt_t as above).  Address a sets bit a mod 64 of word a / 64.
 *  - Invalid k-mers (any non-ACGT base) insert nothing and query false
 *    ([cuSBF] Algorithms 1 and 2, §IV-F).
 *  - Probe k-mers: the i-th output of the SplitMix64 stream seeded with
 *    `seed`, mix(seed + (i+1) * G), shifted right by 64-2k
 *    ([cuSBF] §V-D measures the FPR on uniformly random k-mers).
 *  - Other alphabets ([cuSBF] §IV-A: proteins, 26 symbols of 5 bits; DNA
 *    triplets, 64 symbols of 6 bits spanning 3 bytes): a protein symbol is a
 *    letter A-Z or a-z, code = its place in the alphabet (0..25); a triplet
 *    symbol is the codon at bytes 3j .. 3j+2 (non-overlapping, from the first
 *    byte), code = 16 c0 + 4 c1 + c2 with the DNA codes above, invalid if any
 *    of its bases is.  k-mers, m-mers and s-mers count symbols; a k-mer packs
 *    its symbols first-most-significant at b bits each (b = 2, 5, 6), so
 *    k * b <= 64.  Probe k-mers: triplets take the top 6k bits of the
 *    SplitMix64 output as for DNA; a protein k-mer's symbol j is
 *    floor(26 u / 2^64), u = mix(seed + (i k + j + 1) * G).
 */
#include "sbf_oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull
#define SM_C1 0xBF58476D1CE4E5B9ull
#define SM_C2 0x94D049BB133111EBull

struct osbf {
    int kind;
    unsigned alpha, b; /* alphabet, bits per symbol */
    unsigned k, m, s, H;
    uint64_t num_shards;
    uint64_t* words;
};

/* [cuSBF] §IV-A: DNA, 4 symbols, 2 bits each. */
int osbf_code(unsigned char c)
{
    switch (c) {
    case 'A': case 'a': return 0;
    case 'C': case 'c': return 1;
    case 'G': case 'g': return 2;
    case 'T': case 't': return 3;
    default: return -1;
    }
}

/* [cuSBF] §IV-G: the minimizer hash is a single multiplicative mix. */
uint64_t osbf_hmin(uint64_t v)
{
    uint64_t u = (v + GOLDEN) * SM_C1;
    return u ^ (u >> 32);
}

/* SplitMix64 output function (Steele, Lea, Flood 2014). */
uint64_t osbf_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * SM_C1;
    z = (z ^ (z >> 27)) * SM_C2;
    return z ^ (z >> 31);
}

/* [cuSBF] §IV-G: the s-mer hash is a stronger mix with extra xorshifts. */
uint64_t osbf_hs(uint64_t v)
{
    return osbf_mix(v + GOLDEN);
}

/* [cuSBF] §IV-A: proteins, 26 letters, 5 bits each. */
int osbf_code_protein(unsigned char c)
{
    if (c >= 'A' && c <= 'Z')
        return c - 'A';
    if (c >= 'a' && c <= 'z')
        return c - 'a';
    return -1;
}

/* [cuSBF] §IV-A: DNA triplets, 64 symbols of 6 bits, one codon of 3 bytes. */
int osbf_code_triplet(const char* p)
{
    int c0 = osbf_code((unsigned char)p[0]), c1 = osbf_code((unsigned char)p[1]), c2 = osbf_code((unsigned char)p[2]);
    if (c0 < 0 || c1 < 0 || c2 < 0)
        return -1;
    return 16 * c0 + 4 * c1 + c2;
}

unsigned osbf_symbol_bits(unsigned alpha) { return alpha == OSBF_ALPHA_PROTEIN ? 5u : alpha == OSBF_ALPHA_TRIPLET ? 6u : 2u; }

/* Symbols in a sequence of len bytes. */
static uint64_t n_symbols(unsigned alpha, uint64_t len) { return alpha == OSBF_ALPHA_TRIPLET ? len / 3u : len; }

/* Code of symbol j, or -1 if invalid. */
static int symbol_at(unsigned alpha, const char* seq, uint64_t j)
{
    if (alpha == OSBF_ALPHA_PROTEIN)
        return osbf_code_protein((unsigned char)seq[j]);
    if (alpha == OSBF_ALPHA_TRIPLET)
        return osbf_code_triplet(seq + 3u * j);
    return osbf_code((unsigned char)seq[j]);
}

/* Pack the k symbols starting at symbol p (first most significant, b bits
 * each).  0 and *x on success, -1 if a symbol is invalid. */
int osbf_pack_kmer_alpha(unsigned alpha, const char* seq, uint64_t p, unsigned k, uint64_t* x)
{
    const unsigned b = osbf_symbol_bits(alpha);
    uint64_t v = 0;
    for (unsigned j = 0; j < k; ++j) {
        int c = symbol_at(alpha, seq, p + j);
        if (c < 0)
            return -1;
        v = (v << b) | (uint64_t)c;
    }
    *x = v;
    return 0;
}

/* [cuSBF] §IV-G, bit-slicing and the salted fallback. */
unsigned osbf_bitaddr(uint64_t hs, unsigned t, unsigned H)
{
    if (H <= 10) {
        unsigned width = 64u / H;
        return (unsigned)((hs >> (t * width)) & 63u);
    }
    uint64_t salt = osbf_mix((uint64_t)(t + 1u) * GOLDEN);
    return (unsigned)((hs * salt) >> 58);
}

/* Wide variant: a 9-bit address into a 512-bit block (the CPU reference's
 * whole-block addressing, [cuSBF] §V-D), sliced or salted as above. */
unsigned osbf_bitaddr_wide(uint64_t hs, unsigned t, unsigned H)
{
    if (H <= 7) {
        unsigned width = 64u / H;
        return (unsigned)((hs >> (t * width)) & 511u);
    }
    uint64_t salt = osbf_mix((uint64_t)(t + 1u) * GOLDEN);
    return (unsigned)((hs * salt) >> 55);
}

/* [cuSBF] §V-D: uniformly random k-mers, drawn from SplitMix64. */
uint64_t osbf_probe_kmer(uint64_t seed, uint64_t i, unsigned k)
{
    uint64_t r = osbf_mix(seed + (i + 1ull) * GOLDEN);
    return r >> (64u - 2u * k);
}

/* Probe k-mer i for any alphabet (see the readings above). */
uint64_t osbf_probe_kmer_alpha(unsigned alpha, uint64_t seed, uint64_t i, unsigned k)
{
    if (alpha == OSBF_ALPHA_PROTEIN) {
        uint64_t x = 0;
        for (unsigned j = 0; j < k; ++j) {
            uint64_t u = osbf_mix(seed + ((uint64_t)i * k + j + 1ull) * GOLDEN);
            x = (x << 5) | (uint64_t)(((unsigned __int128)u * 26u) >> 64);
        }
        return x;
    }
    const unsigned bits = osbf_symbol_bits(alpha) * k;
    uint64_t r = osbf_mix(seed + (i + 1ull) * GOLDEN);
    return bits >= 64 ? r : r >> (64u - bits);
}

static uint64_t low_mask(unsigned nbases)
{
    return nbases >= 32 ? ~0ull : ((1ull << (2u * nbases)) - 1ull);
}

/* Window of w symbols starting at symbol i of a packed k-mer, b bits each. */
static uint64_t sub_b(uint64_t x, unsigned k, unsigned i, unsigned w, unsigned b)
{
    const unsigned bits = b * w;
    return (x >> (b * (k - w - i))) & (bits >= 64 ? ~0ull : ((1ull << bits) - 1ull));
}

/* [cuSBF] §IV-C: pack k symbols into one 64-bit word by shift-and-OR. */
int osbf_pack_kmer(const char* seq, unsigned k, uint64_t* x)
{
    uint64_t v = 0;
    for (unsigned j = 0; j < k; ++j) {
        int c = osbf_code((unsigned char)seq[j]);
        if (c < 0)
            return -1;
        v = (v << 2) | (uint64_t)c;
    }
    *x = v;
    return 0;
}

/* Window of w bases starting at base i of a packed k-mer. */
uint64_t osbf_subwindow(uint64_t x, unsigned k, unsigned i, unsigned w)
{
    return (x >> (2u * (k - w - i))) & low_mask(w);
}

/* [cuSBF] §II-B-1 and Algorithm 1: the minimizer is the m-mer of least hash;
 * the shard only needs that least hash value. */
uint64_t osbf_minimizer_hash(uint64_t x, unsigned k, unsigned m)
{
    uint64_t best = ~0ull;
    for (unsigned i = 0; i + m <= k; ++i) {
        uint64_t h = osbf_hmin(osbf_subwindow(x, k, i, m));
        if (h < best)
            best = h;
    }
    return best;
}

/* Minimizer hash of every k-mer start of an ASCII DNA sequence, each from
 * its own packed k-mer (no sliding): out[p] for p in [0, len-k+1), ~0 for an
 * invalid k-mer.  Returns the number of valid k-mers.  For density checks of
 * the minimizer scheme ([cuSBF] §II-B-1) on long random text. */
uint64_t osbf_minimizer_hashes(const char* seq, uint64_t len, unsigned k, unsigned m, uint64_t* out)
{
    uint64_t valid = 0;
    if (len < k)
        return 0;
    for (uint64_t p = 0; p + k <= len; ++p) {
        uint64_t x;
        if (osbf_pack_kmer(seq + p, k, &x) == 0) {
            out[p] = osbf_minimizer_hash(x, k, m);
            ++valid;
        } else {
            out[p] = ~0ull;
        }
    }
    return valid;
}

osbf* osbf_create(int kind, unsigned k, unsigned m, unsigned s, unsigned H, uint64_t bits)
{
    return osbf_create_alpha(kind, OSBF_ALPHA_DNA, k, m, s, H, bits);
}

osbf* osbf_create_alpha(int kind, unsigned alpha, unsigned k, unsigned m, unsigned s, unsigned H, uint64_t bits)
{
    if (kind != OSBF_KIND_SBF && kind != OSBF_KIND_BBF && kind != OSBF_KIND_WIDE)
        return NULL;
    if (alpha > OSBF_ALPHA_TRIPLET)
        return NULL;
    if (k < 1 || k * osbf_symbol_bits(alpha) > 64 || H < 1 || H > 64 || bits < 1)
        return NULL;
    if (kind != OSBF_KIND_BBF && (m < 1 || m > k || s < 1 || s > k))
        return NULL;
    /* [cuSBF] §IV-B: shard count rounded up to a power of two. */
    const uint64_t block = kind == OSBF_KIND_WIDE ? 512u : 256u;
    uint64_t need = bits / block + (bits % block != 0);
    uint64_t n = 1;
    while (n < need)
        n <<= 1;
    osbf* f = (osbf*)calloc(1, sizeof(osbf));
    if (!f)
        return NULL;
    f->words = (uint64_t*)calloc((block / 64u) * n, sizeof(uint64_t));
    if (!f->words) {
        free(f);
        return NULL;
    }
    f->kind = kind;
    f->alpha = alpha;
    f->b = osbf_symbol_bits(alpha);
    f->k = k;
    f->m = m;
    f->s = s;
    f->H = H;
    f->num_shards = n;
    return f;
}

void osbf_destroy(osbf* f)
{
    if (!f)
        return;
    free(f->words);
    free(f);
}

uint64_t osbf_num_shards(const osbf* f) { return f->num_shards; }
unsigned osbf_words_per_shard(const osbf* f) { return f->kind == OSBF_KIND_WIDE ? 8u : 4u; }
uint64_t* osbf_words(osbf* f) { return f->words; }

/* SBF: [cuSBF] Algorithm 1, shard = minimizer hash & (N-1).
 * BBF: [cuSBF] §II-A / Fig. 1b, one hash of the whole key picks the block. */
uint64_t osbf_shard_of(const osbf* f, uint64_t x)
{
    if (f->kind == OSBF_KIND_BBF)
        return osbf_hs(x) & (f->num_shards - 1u);
    uint64_t best = ~0ull;
    for (unsigned i = 0; i + f->m <= f->k; ++i) {
        uint64_t h = osbf_hmin(sub_b(x, f->k, i, f->m, f->b));
        if (h < best)
            best = h;
    }
    return best & (f->num_shards - 1u);
}

/* [cuSBF] §IV-B: hash index t sets one bit in word t mod 4 of the shard;
 * wide variant: bit a mod 64 of word a / 64 for its 9-bit address a. */
static void set_bits(const osbf* f, uint64_t* shard, uint64_t hs)
{
    for (unsigned t = 0; t < f->H; ++t) {
        if (f->kind == OSBF_KIND_WIDE) {
            unsigned a = osbf_bitaddr_wide(hs, t, f->H);
            shard[a / 64u] |= 1ull << (a % 64u);
        } else {
            shard[t % 4u] |= 1ull << osbf_bitaddr(hs, t, f->H);
        }
    }
}

static int test_bits(const osbf* f, const uint64_t* shard, uint64_t hs)
{
    for (unsigned t = 0; t < f->H; ++t) {
        if (f->kind == OSBF_KIND_WIDE) {
            unsigned a = osbf_bitaddr_wide(hs, t, f->H);
            if (!((shard[a / 64u] >> (a % 64u)) & 1u))
                return 0;
        } else if (!((shard[t % 4u] >> osbf_bitaddr(hs, t, f->H)) & 1u)) {
            return 0;
        }
    }
    return 1;
}

/* [cuSBF] §II-B-2 (Findere) and Algorithm 1: every one of the k-s+1 s-mers
 * sets its H bits in the k-mer's shard.  The BBF keys its bits on a second
 * hash of the k-mer's block hash. */
void osbf_insert_kmer(osbf* f, uint64_t x)
{
    uint64_t* shard = f->words + osbf_words_per_shard(f) * osbf_shard_of(f, x);
    if (f->kind == OSBF_KIND_BBF) {
        set_bits(f, shard, osbf_hs(osbf_hs(x)));
        return;
    }
    for (unsigned j = 0; j + f->s <= f->k; ++j)
        set_bits(f, shard, osbf_hs(sub_b(x, f->k, j, f->s, f->b)));
}

/* [cuSBF] §II-B-2 and Algorithm 2 (Contains): present only if every s-mer
 * finds all of its H bits. */
int osbf_query_kmer(const osbf* f, uint64_t x)
{
    const uint64_t* shard = f->words + osbf_words_per_shard(f) * osbf_shard_of(f, x);
    if (f->kind == OSBF_KIND_BBF)
        return test_bits(f, shard, osbf_hs(osbf_hs(x)));
    for (unsigned j = 0; j + f->s <= f->k; ++j)
        if (!test_bits(f, shard, osbf_hs(sub_b(x, f->k, j, f->s, f->b))))
            return 0;
    return 1;
}

/* [cuSBF] §IV-D / §IV-F: every k-mer start; invalid k-mers are skipped. */
void osbf_insert_seq(osbf* f, const char* seq, uint64_t len)
{
    const uint64_t ns = n_symbols(f->alpha, len);
    if (ns < f->k)
        return;
    for (uint64_t p = 0; p + f->k <= ns; ++p) {
        uint64_t x;
        if (osbf_pack_kmer_alpha(f->alpha, seq, p, f->k, &x) == 0)
            osbf_insert_kmer(f, x);
    }
}

/* [cuSBF] §IV-E: one answer per k-mer start, invalid k-mers answer false. */
void osbf_query_seq(const osbf* f, const char* seq, uint64_t len, uint64_t* out)
{
    const uint64_t ns = n_symbols(f->alpha, len);
    if (ns < f->k)
        return;
    uint64_t nk = ns - f->k + 1u;
    memset(out, 0, ((nk + 63u) / 64u) * sizeof(uint64_t));
    for (uint64_t p = 0; p < nk; ++p) {
        uint64_t x;
        if (osbf_pack_kmer_alpha(f->alpha, seq, p, f->k, &x) == 0 && osbf_query_kmer(f, x))
            out[p / 64u] |= 1ull << (p % 64u);
    }
}

void osbf_query_positions(const osbf* f, const char* seq, uint64_t len,
                          const uint64_t* pos, uint64_t n, uint8_t* out)
{
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t x;
        uint64_t p = pos[i];
        out[i] = 0;
        if (p + f->k <= n_symbols(f->alpha, len) && osbf_pack_kmer_alpha(f->alpha, seq, p, f->k, &x) == 0)
            out[i] = (uint8_t)osbf_query_kmer(f, x);
    }
}

/* [cuSBF] §V-D: count positives among n random k-mers. */
uint64_t osbf_fpr_probe(const osbf* f, uint64_t n, uint64_t seed)
{
    uint64_t hits = 0;
    for (uint64_t i = 0; i < n; ++i)
        hits += (uint64_t)osbf_query_kmer(f, osbf_probe_kmer_alpha(f->alpha, seed, i, f->k));
    return hits;
}

/* ---- multi-threaded drivers ------------------------------------------------
 * The same per-k-mer definition, with the k-mer starts split into contiguous
 * ranges over threads.  Insert ORs bits with atomic fetch-or into the one
 * filter (OR is commutative and idempotent, so the result is the
 * single-threaded one); query ranges are whole 64-bit answer words, so the
 * threads write disjoint words.  Used only to check large inputs. */

typedef struct {
    osbf* f;
    const char* seq;
    uint64_t len, p0, p1;
    uint64_t* out;
    uint64_t* checked;               /* sampled query: positions that were checked */
    uint64_t sample_mask, sample_value; /* shards with (shard & mask) == value */
} osbf_job;

static void set_bits_atomic(const osbf* f, uint64_t* shard, uint64_t hs)
{
    for (unsigned t = 0; t < f->H; ++t) {
        if (f->kind == OSBF_KIND_WIDE) {
            unsigned a = osbf_bitaddr_wide(hs, t, f->H);
            __atomic_fetch_or(&shard[a / 64u], 1ull << (a % 64u), __ATOMIC_RELAXED);
        } else {
            __atomic_fetch_or(&shard[t % 4u], 1ull << osbf_bitaddr(hs, t, f->H), __ATOMIC_RELAXED);
        }
    }
}

static void* insert_worker(void* arg)
{
    osbf_job* j = (osbf_job*)arg;
    osbf* f = j->f;
    for (uint64_t p = j->p0; p < j->p1; ++p) {
        uint64_t x;
        if (osbf_pack_kmer_alpha(f->alpha, j->seq, p, f->k, &x) != 0)
            continue;
        uint64_t sh = osbf_shard_of(f, x);
        if ((sh & j->sample_mask) != j->sample_value)
            continue;
        uint64_t* shard = f->words + osbf_words_per_shard(f) * sh;
        if (f->kind == OSBF_KIND_BBF) {
            set_bits_atomic(f, shard, osbf_hs(osbf_hs(x)));
            continue;
        }
        for (unsigned s = 0; s + f->s <= f->k; ++s)
            set_bits_atomic(f, shard, osbf_hs(sub_b(x, f->k, s, f->s, f->b)));
    }
    return NULL;
}

static void* query_worker(void* arg)
{
    osbf_job* j = (osbf_job*)arg;
    for (uint64_t p = j->p0; p < j->p1; ++p) {
        uint64_t x;
        if (osbf_pack_kmer_alpha(j->f->alpha, j->seq, p, j->f->k, &x) != 0)
            continue;
        if (j->checked) {
            if ((osbf_shard_of(j->f, x) & j->sample_mask) != j->sample_value)
                continue;
            j->checked[p / 64u] |= 1ull << (p % 64u);
        }
        if (osbf_query_kmer(j->f, x))
            j->out[p / 64u] |= 1ull << (p % 64u);
    }
    return NULL;
}

static void run_jobs(osbf* f, const char* seq, uint64_t len, uint64_t* out, uint64_t* checked,
                     uint64_t sample_mask, uint64_t sample_value, unsigned nthreads, void* (*fn)(void*))
{
    uint64_t nk = n_symbols(f->alpha, len) - f->k + 1u;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    osbf_job jobs[256];
    pthread_t th[256];
    uint64_t chunk = (nk + nthreads - 1) / nthreads;
    chunk = (chunk + 63u) & ~63ull; /* whole answer words per thread */
    unsigned started = 0;
    for (unsigned t = 0; t < nthreads; ++t) {
        uint64_t p0 = (uint64_t)t * chunk, p1 = p0 + chunk;
        if (p0 >= nk)
            break;
        if (p1 > nk)
            p1 = nk;
        jobs[t].f = f;
        jobs[t].seq = seq;
        jobs[t].len = len;
        jobs[t].p0 = p0;
        jobs[t].p1 = p1;
        jobs[t].out = out;
        jobs[t].checked = checked;
        jobs[t].sample_mask = sample_mask;
        jobs[t].sample_value = sample_value;
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) {
            fn(&jobs[t]); /* run inline if a thread cannot start */
            th[t] = 0;
        }
        ++started;
    }
    for (unsigned t = 0; t < started; ++t)
        if (th[t])
            pthread_join(th[t], NULL);
}

void osbf_insert_seq_mt(osbf* f, const char* seq, uint64_t len, unsigned nthreads)
{
    if (n_symbols(f->alpha, len) < f->k)
        return;
    run_jobs(f, seq, len, NULL, NULL, 0, 0, nthreads, insert_worker);
}

void osbf_query_seq_mt(const osbf* f, const char* seq, uint64_t len, uint64_t* out, unsigned nthreads)
{
    if (n_symbols(f->alpha, len) < f->k)
        return;
    uint64_t nk = n_symbols(f->alpha, len) - f->k + 1u;
    memset(out, 0, ((nk + 63u) / 64u) * sizeof(uint64_t));
    run_jobs((osbf*)f, seq, len, out, NULL, 0, 0, nthreads, query_worker);
}

/* Shard-sampled insert: only k-mers whose shard satisfies
 * (shard & sample_mask) == sample_value; the words of those shards then
 * equal the full insert's exactly, every other shard stays empty. */
void osbf_insert_seq_sampled_mt(osbf* f, const char* seq, uint64_t len, uint64_t sample_mask,
                                uint64_t sample_value, unsigned nthreads)
{
    if (n_symbols(f->alpha, len) < f->k)
        return;
    run_jobs(f, seq, len, NULL, NULL, sample_mask, sample_value, nthreads, insert_worker);
}

/* Query restricted to the sampled shards: checked bit p = valid k-mer p maps
 * to a sampled shard; out bit p = its answer (0 where not checked). */
void osbf_query_seq_sampled_mt(const osbf* f, const char* seq, uint64_t len, uint64_t* out, uint64_t* checked,
                               uint64_t sample_mask, uint64_t sample_value, unsigned nthreads)
{
    if (n_symbols(f->alpha, len) < f->k)
        return;
    uint64_t nk = n_symbols(f->alpha, len) - f->k + 1u;
    memset(out, 0, ((nk + 63u) / 64u) * sizeof(uint64_t));
    memset(checked, 0, ((nk + 63u) / 64u) * sizeof(uint64_t));
    run_jobs((osbf*)f, seq, len, out, checked, sample_mask, sample_value, nthreads, query_worker);
}
