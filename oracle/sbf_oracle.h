/*
 * sbf_oracle.h -- plain, single-threaded CPU oracle of the Super Bloom filter.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously correct definition
 * that the GPU library is checked against.  Only the test suite, the smoke
 * entry point and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant generator with the HIP library.
 *
 * Source: "cuSBF: A Minimizer-Aware Bloom Filter for Genomic Sequence Data
 * on Modern GPUs" (Dortmann, Vieth, Schmidt), referred to below as [cuSBF].
 *
 * Every operation is written per k-mer, straight from its definition: no
 * sliding windows, no run grouping, no batching.  Insert is a set union and
 * query a pure function of (k-mer, filter), so this per-k-mer loop fixes the
 * one correct result for any input.
 *
 * Fixed readings where [cuSBF] is silent (hash constants, code order, bit
 * order) are listed at the top of sbf_oracle.c.
 */
#ifndef SBF_ORACLE_H
#define SBF_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* kind of filter */
#define OSBF_KIND_SBF 0 /* Super Bloom filter (minimizer shard + Findere s-mers) */
#define OSBF_KIND_BBF 1 /* per-k-mer blocked Bloom filter with the same shard layout */
#define OSBF_KIND_WIDE 2 /* SBF with 512-bit blocks, each hash addressing the whole block */

/* alphabet of the sequences ([cuSBF] §IV-A) */
#define OSBF_ALPHA_DNA 0     /* A C G T, 2 bits per symbol */
#define OSBF_ALPHA_PROTEIN 1 /* letters A-Z, 5 bits per symbol */
#define OSBF_ALPHA_TRIPLET 2 /* non-overlapping DNA codons, 6 bits per symbol */

typedef struct osbf osbf;

/* ---- primitives (exposed for the pins) ---------------------------------- */

/* 2-bit code of one base, or -1 if the byte is not a DNA base. */
int osbf_code(unsigned char c);
/* minimizer hash h_min and s-mer hash h_s; mix is the SplitMix64 finalizer */
uint64_t osbf_hmin(uint64_t v);
uint64_t osbf_mix(uint64_t z);
uint64_t osbf_hs(uint64_t v);
/* bit position (0..63) of hash index t of an s-mer hash, for H hashes */
unsigned osbf_bitaddr(uint64_t hs, unsigned t, unsigned H);
/* wide variant: bit position (0..511) in the 512-bit block */
unsigned osbf_bitaddr_wide(uint64_t hs, unsigned t, unsigned H);
/* i-th probe k-mer (0-based) of the stream started at `seed` */
uint64_t osbf_probe_kmer(uint64_t seed, uint64_t i, unsigned k);

/* protein code 0..25 of a letter (either case), or -1 */
int osbf_code_protein(unsigned char c);
/* triplet code 16 c0 + 4 c1 + c2 of the codon at p[0..2], or -1 */
int osbf_code_triplet(const char* p);
/* bits per symbol: 2, 5 or 6 */
unsigned osbf_symbol_bits(unsigned alpha);
/* Pack the k symbols starting at symbol p of seq (for triplets symbol j is
 * bytes 3j..3j+2), first most significant, b bits each.  0 and *x, or -1 if
 * a symbol is invalid. */
int osbf_pack_kmer_alpha(unsigned alpha, const char* seq, uint64_t p, unsigned k, uint64_t* x);
/* i-th probe k-mer for an alphabet (DNA: osbf_probe_kmer) */
uint64_t osbf_probe_kmer_alpha(unsigned alpha, uint64_t seed, uint64_t i, unsigned k);

/* Pack k bases starting at seq into a k-mer value, first base most
 * significant.  Returns 0 and sets *x if every base is valid, else -1. */
int osbf_pack_kmer(const char* seq, unsigned k, uint64_t* x);
/* value of the i-th sub-window of length w of a packed k-mer (0 = first) */
uint64_t osbf_subwindow(uint64_t x, unsigned k, unsigned i, unsigned w);
/* minimizer hash of a packed k-mer: min over its k-m+1 m-mers of h_min */
uint64_t osbf_minimizer_hash(uint64_t x, unsigned k, unsigned m);

/* minimizer hash of every k-mer start of an ASCII DNA sequence (out[p] for
 * p < len-k+1, ~0 where the k-mer is invalid); returns the valid count */
uint64_t osbf_minimizer_hashes(const char* seq, uint64_t len, unsigned k, unsigned m, uint64_t* out);

/* ---- filter ------------------------------------------------------------- */

/* Returns NULL on invalid parameters or allocation failure. */
osbf* osbf_create(int kind, unsigned k, unsigned m, unsigned s, unsigned H, uint64_t bits);
/* The same for an alphabet; k, m and s count symbols, k * b <= 64.  The
 * sequence calls below then take symbol positions: for triplets a sequence of
 * len bytes holds floor(len / 3) symbols. */
osbf* osbf_create_alpha(int kind, unsigned alpha, unsigned k, unsigned m, unsigned s, unsigned H, uint64_t bits);
void osbf_destroy(osbf* f);
uint64_t osbf_num_shards(const osbf* f);
/* 4, or 8 for the wide variant */
unsigned osbf_words_per_shard(const osbf* f);
/* the filter: W * num_shards words (W = words per shard), shard j is words
 * Wj .. Wj+W-1 */
uint64_t* osbf_words(osbf* f);

/* shard a packed k-mer maps to */
uint64_t osbf_shard_of(const osbf* f, uint64_t x);
/* insert / test one packed k-mer */
void osbf_insert_kmer(osbf* f, uint64_t x);
int osbf_query_kmer(const osbf* f, uint64_t x);

/* Insert every valid k-mer of an ASCII sequence. */
void osbf_insert_seq(osbf* f, const char* seq, uint64_t len);
/* Query every k-mer start of an ASCII sequence.  out receives
 * ceil((len-k+1)/64) words; bit p (LSB-first within word p/64) is the answer
 * for the k-mer starting at p; invalid k-mers and tail bits are 0.
 * Nothing is written when len < k. */
void osbf_query_seq(const osbf* f, const char* seq, uint64_t len, uint64_t* out);
/* Query the k-mers starting at the given positions; out[i] = 0/1. */
void osbf_query_positions(const osbf* f, const char* seq, uint64_t len,
                          const uint64_t* pos, uint64_t n, uint8_t* out);
/* Number of positives among n probe k-mers from the stream at `seed`. */
uint64_t osbf_fpr_probe(const osbf* f, uint64_t n, uint64_t seed);

/* The same insert and query with the k-mer starts split over threads (for
 * checking large inputs); results equal the single-threaded calls. */
void osbf_insert_seq_mt(osbf* f, const char* seq, uint64_t len, unsigned nthreads);
void osbf_query_seq_mt(const osbf* f, const char* seq, uint64_t len, uint64_t* out, unsigned nthreads);
/* Shard-sampled variants: only k-mers whose shard s has
 * (s & sample_mask) == sample_value take part.  The sampled shards' words
 * then equal those of the full insert; checked marks the queried k-mers. */
void osbf_insert_seq_sampled_mt(osbf* f, const char* seq, uint64_t len, uint64_t sample_mask,
                                uint64_t sample_value, unsigned nthreads);
void osbf_query_seq_sampled_mt(const osbf* f, const char* seq, uint64_t len, uint64_t* out, uint64_t* checked,
                               uint64_t sample_mask, uint64_t sample_value, unsigned nthreads);

#ifdef __cplusplus
}
#endif
#endif
