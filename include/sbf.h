/*
 * sbf.h -- C ABI of the MI355X (gfx950) Super Bloom filter library, libsbf.so.
 *
 * The method is that of "cuSBF: A Minimizer-Aware Bloom Filter for Genomic
 * Sequence Data on Modern GPUs" (Dortmann, Vieth, Schmidt), cited as [cuSBF]:
 * DNA is 2-bit packed; the minimizer hash of each k-mer picks one 256-bit
 * shard (§II-B-1, §IV-B); each of the k-mer's k-s+1 overlapping s-mers sets
 * or tests H bits inside that shard, hash index t in 64-bit word t mod 4
 * (Findere, §II-B-2; §IV-B); a k-mer is present only if all of its s-mers
 * hit (Algorithm 2).  Hash functions and bit orders are fixed as follows:
 *
 *   codes        A/a=0 C/c=1 G/g=2 T/t=3, every other byte is invalid
 *   k-mer value  first base in the most significant bits (§IV-C)
 *   h_min(v)     u ^ (u >> 32), u = (v + G) * C1 mod 2^64       (§IV-G)
 *   h_s(v)       SplitMix64 finalizer of v + G                   (§IV-G)
 *   bit of hash t: H <= 10: bits [t*floor(64/H), +6) of h_s;
 *                  H > 10 : top 6 bits of h_s * S_t,             (§IV-G)
 *                           S_t = SplitMix64 finalizer of (t+1) * G
 *   shard        min over the k-m+1 m-mers of h_min, & (N-1)     (Algorithm 1)
 *   N            smallest power of two >= ceil(bits / 256)       (§IV-B)
 *   G = 0x9E3779B97F4A7C15, C1 = 0xBF58476D1CE4E5B9, C2 = 0x94D049BB133111EB
 *
 * Conventions
 *  - Every call returns SBF_OK (0) or a negative SBF_E* code and never aborts.
 *    A failing call leaves no partial allocation behind; the text of the last
 *    error of the calling thread is returned by sbf_last_error().
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Calls flagged SBF_HOST take host pointers and synchronize before they
 *    return; calls flagged SBF_DEVICE (and the *_packed / *_device calls) take
 *    device pointers and are asynchronous on `stream` ([cuSBF] §IV-A: host
 *    entry points synchronize, device entry points leave ordering to the
 *    caller).
 *  - Concurrent inserts into one filter are safe (bitwise OR is idempotent and
 *    commutative), but calls on one handle share its staging buffers: issue
 *    the *_seq calls of one handle on one stream, or serialize them.
 *
 * Packed sequence layout (device memory), for a sequence of `len` bases:
 *  - codes: uint32_t[ceil(len/16)]; base j occupies bits 31-2r..30-2r of word
 *    j/16, r = j mod 16 (the first base of a word is in its top bits).
 *  - valid: uint32_t[ceil(len/32)]; bit j mod 32 of word j/32 is 1 iff base j
 *    is one of ACGTacgt.  Bits at or beyond len must be 0 (sbf_pack writes
 *    them so); k-mers that would reach past len are never valid.
 * Query output: uint64_t[ceil((len-k+1)/64)]; bit p mod 64 of word p/64 is the
 * answer for the k-mer starting at base p (LSB first); invalid k-mers and the
 * bits past len-k+1 are 0.  Nothing is written when len < k.
 */
#ifndef SBF_H
#define SBF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define SBF_OK 0
#define SBF_EINVAL (-1)       /* bad argument (parameter range, NULL pointer, size) */
#define SBF_EUNSUPPORTED (-2) /* call not available for this filter (see sbf_create_alphabet) */
#define SBF_ENOMEM (-3)       /* device or host allocation failed */
#define SBF_EDEVICE (-4)      /* a HIP runtime call or kernel launch failed */
#define SBF_EIO (-5)          /* a file could not be opened or read, or is not valid FASTA/FASTQ */

/* filter kinds */
#define SBF_KIND_SBF 0 /* Super Bloom filter */
#define SBF_KIND_BBF 1 /* per-k-mer blocked Bloom filter, same shard layout */
#define SBF_KIND_WIDE 2 /* Super Bloom filter with 512-bit blocks, whole-block addressing */

/* sequence alphabets ([cuSBF] §IV-A) */
#define SBF_ALPHABET_DNA 0u     /* A C G T, 2 bits per symbol */
#define SBF_ALPHABET_PROTEIN 1u /* letters A-Z, 5 bits per symbol */
#define SBF_ALPHABET_TRIPLET 2u /* DNA codons of 3 bytes, 6 bits per symbol */

/* where the pointers of a *_seq / copy call live */
#define SBF_HOST 1u
#define SBF_DEVICE 2u

typedef struct sbf_handle sbf_t;

typedef struct sbf_info {
    uint32_t k, m, s, H; /* m = s = 0 for a blocked Bloom filter */
    uint32_t kind;       /* SBF_KIND_* */
    uint32_t specialized; /* 1 if a compile-time specialized kernel set serves it */
    uint64_t num_shards;  /* N, a power of two */
    uint64_t filter_bytes; /* 8 * words_per_shard * N */
    uint32_t words_per_shard; /* 4, or 8 for SBF_KIND_WIDE */
    uint32_t alphabet;        /* SBF_ALPHABET_* */
} sbf_info_t;

/*
 * Create an empty Super Bloom filter ([cuSBF] §IV-A: k, s, m, H fix the
 * method, the filter size in bits is the only run-time input; §IV-B layout).
 * Requires 1 <= m <= k <= 32, 1 <= s <= k, 1 <= H <= 64, 1 <= bits <= 2^40.
 * The device filter (uint64_t[4N], zeroed) is owned by the handle; *out is
 * set only on success.  Errors: SBF_EINVAL, SBF_ENOMEM, SBF_EDEVICE.
 */
int sbf_create(sbf_t** out, uint32_t k, uint32_t m, uint32_t s, uint32_t H, uint64_t bits);

/*
 * Create an empty per-k-mer blocked Bloom filter ([cuSBF] §II-A, Fig. 1b):
 * block = h_s(x) & (N-1), hash t sets bit t of h_s(h_s(x)) (sliced as above)
 * in word t mod 4 of the block.  Same shard layout and calls as the SBF.
 * Requires 1 <= k <= 32, 1 <= H <= 64, 1 <= bits <= 2^40.
 */
int sbf_create_bbf(sbf_t** out, uint32_t k, uint32_t H, uint64_t bits);

/*
 * Create an empty wide-block Super Bloom filter: the layout [cuSBF] §V-D
 * attributes to the CPU Super Bloom reference.  Shards are 512-bit blocks
 * (uint64_t[8N], N = smallest power of two >= ceil(bits / 512)), chosen by
 * the minimizer as above; hash index t of an s-mer hash h_s addresses any of
 * the block's 512 bits: a = bits [t*floor(64/H), +9) of h_s for H <= 7, the
 * top 9 bits of h_s * S_t for H > 7; it sets bit a mod 64 of word a / 64.
 * Same calls and parameter ranges as sbf_create; shard j of the copied filter
 * is words 8j .. 8j+7.
 */
int sbf_create_wide(sbf_t** out, uint32_t k, uint32_t m, uint32_t s, uint32_t H, uint64_t bits);

/*
 * Create an empty Super Bloom filter over another alphabet ([cuSBF] §IV-A:
 * proteins, 26 symbols of 5 bits; DNA triplets, 64 symbols of 6 bits that
 * span three bytes).  k, m and s count symbols and a k-mer packs its symbols
 * first-most-significant at b bits each, so k * b <= 64: k <= 12 for
 * proteins, k <= 10 for triplets (DNA: k <= 32, the same as sbf_create).
 * Symbol codes:
 *   protein  a letter of either case -> its place in A..Z (0..25); every other
 *            byte is invalid
 *   triplet  symbol j is bytes 3j .. 3j+2 (non-overlapping, from the first
 *            byte; a last 1 or 2 bytes are ignored), code 16 c0 + 4 c1 + c2
 *            with the DNA codes; invalid if any of its bases is
 * Shard, s-mer bits and layout are those of sbf_create with symbols in place
 * of bases.  On a protein or triplet filter, positions in the sequence calls
 * are symbol positions: a sequence of len bytes has n = len (protein) or
 * floor(len / 3) (triplet) symbols, n - k + 1 k-mer starts, and query output
 * has ceil((n - k + 1) / 64) words.  sbf_insert_seq, sbf_query_seq (host or
 * device), sbf_fpr_probe* (protein probe symbol j of k-mer i is
 * floor(26 u / 2^64), u the SplitMix64 output number i*k + j + 1 of the seed;
 * triplet probes take the top 6k bits of output i + 1), sbf_clear, sbf_info
 * and sbf_copy_filter work as for DNA; the packed and FASTA/FASTQ calls
 * return SBF_EUNSUPPORTED.  alphabet = SBF_ALPHABET_DNA is sbf_create.
 * Errors: SBF_EINVAL (unknown alphabet, parameter ranges), SBF_ENOMEM,
 * SBF_EDEVICE.
 */
int sbf_create_alphabet(sbf_t** out, uint32_t alphabet, uint32_t k, uint32_t m, uint32_t s, uint32_t H,
                        uint64_t bits);

/*
 * Free a filter and its buffers (synchronizes the device).  NULL is a no-op.
 * Not an operation of the method: [cuSBF] §IV-A describes the filter as a
 * device object built from (k, m, s, H) and a size, and says nothing of its
 * release; here the handle owns its device memory until this call.
 * Errors: SBF_EDEVICE if the synchronization reports an earlier failure (the
 * memory is freed all the same).
 */
int sbf_destroy(sbf_t* h);

/*
 * Zero the filter, asynchronously on `stream`: the empty filter of [cuSBF]
 * §IV-B (every bit of every shard 0), as sbf_create leaves it.  The page
 * defines no clear; a filter is refilled by clearing and inserting again.
 * Errors: SBF_EINVAL for a NULL handle, SBF_EDEVICE if the launch fails.
 */
int sbf_clear(sbf_t* h, void* stream);

/*
 * Parameters and sizes of a filter into a caller-owned struct: (k, m, s, H)
 * of [cuSBF] §IV-A and the shard count after the rounding to a power of two
 * of §IV-B (the page fixes the sizes; it defines no call that reports them).
 * Host only, no device work.  Errors: SBF_EINVAL for a NULL argument.
 */
int sbf_info(const sbf_t* h, sbf_info_t* out);

/*
 * Copy the raw filter words (uint64_t[W*N], shard j = words Wj..Wj+W-1, W =
 * words_per_shard) to dst: the bit array in the shard and sector layout of
 * [cuSBF] §IV-B (word 4j+q is sector q of shard j; the page defines the
 * layout, not a copy of it -- this exists for inspection and parity checks).
 * flags = SBF_HOST: dst is host memory, synchronizes; SBF_DEVICE: device
 * memory, asynchronous on `stream`.  The caller owns dst.  SBF_EINVAL for a
 * NULL argument, other flags, or bytes < 8 * W * N; SBF_EDEVICE if the copy
 * fails.
 */
int sbf_copy_filter(const sbf_t* h, void* dst, uint64_t bytes, uint32_t flags, void* stream);

/*
 * Device pointer to the filter words in the layout of sbf_copy_filter
 * ([cuSBF] §IV-B; the page defines no such accessor).  Owned by the handle,
 * valid until sbf_destroy; writing through it changes the filter.  NULL for a
 * NULL handle; no device work, no error code.
 */
const uint64_t* sbf_filter_device_ptr(const sbf_t* h);

/* Number of uint32_t words of the packed codes and validity of len bases, in
 * the packed layout above (2 bits per base, [cuSBF] §IV-A; the storage order
 * is this library's).  Host only; NULL outputs are skipped. */
void sbf_packed_words(uint64_t len, uint64_t* code_words, uint64_t* valid_words);

/*
 * Pack an ASCII sequence held in device memory into the layout above
 * ([cuSBF] §IV-A 2-bit DNA alphabet, §IV-F: any non-ACGT byte -- an 'N'
 * separator between records, a newline -- is invalid).  Asynchronous.  The
 * caller allocates both outputs (sbf_packed_words).  len = 0 is a no-op.
 */
int sbf_pack(const char* d_ascii, uint64_t len, uint32_t* d_codes, uint32_t* d_valid, void* stream);

/*
 * Insert every valid k-mer of a packed device sequence ([cuSBF] §IV-D,
 * Algorithm 1).  Asynchronous on `stream`; len < k is a no-op.  DNA filters
 * only (SBF_EUNSUPPORTED otherwise), as is sbf_query_packed.
 */
int sbf_insert_packed(sbf_t* h, const uint32_t* d_codes, const uint32_t* d_valid,
                      uint64_t len, void* stream);

/*
 * Query every k-mer start of a packed device sequence ([cuSBF] §IV-E,
 * Algorithm 2) into d_out (device, ceil((len-k+1)/64) words, fully
 * overwritten).  Asynchronous.  len < k is a no-op.
 */
int sbf_query_packed(sbf_t* h, const uint32_t* d_codes, const uint32_t* d_valid,
                     uint64_t len, uint64_t* d_out, void* stream);

/*
 * Sequence-native insert ([cuSBF] §IV-A input forms, §IV-F records joined by
 * an invalid separator).  flags = SBF_HOST: `seq` is host memory; it goes
 * through the handle's host pipeline ([cuSBF] §IV-G host staging): chunks of
 * up to sbf_set_staging() k-mer starts (consecutive chunks overlap by k-1
 * bases) are copied into pinned buffers, sent to the device and packed and
 * inserted on three rotating streams, so the host fills one chunk while the
 * copies and kernels of the others run; the work is ordered after earlier
 * work on `stream`
 * and the call synchronizes.  SBF_DEVICE: `seq` is device memory; packing
 * goes to the handle's staging buffer and the call is asynchronous on
 * `stream`, except that a DNA filter with a compiled parameter set reads a
 * 16-byte-aligned device sequence as ASCII in the insert kernel itself (no
 * packing pass, no staging; the same filter for any alignment).  Staging
 * buffers grow on demand (growing synchronizes `stream`) and stay allocated
 * until sbf_destroy.  Protein and triplet filters read the text itself (no
 * packing; chunks overlap by k-1 symbols).
 */
int sbf_insert_seq(sbf_t* h, const char* seq, uint64_t len, uint32_t flags, void* stream);

/*
 * Sequence-native query: one bit per k-mer start into out_bits
 * (ceil((len-k+1)/64) uint64_t words, fully overwritten), which lives where
 * `flags` says (SBF_HOST: synchronizes; SBF_DEVICE: asynchronous).  Input and
 * staging as for sbf_insert_seq, except that a DNA filter whose query takes
 * 32 k-mers per lane (k-s+1 <= 8 and k-m+1 >= 12) reads a 16-byte-aligned
 * device sequence, and each host chunk, as ASCII in the query kernel itself:
 * no packing pass and no staging buffer.  The answers are the same for any
 * alignment.
 */
int sbf_query_seq(sbf_t* h, const char* seq, uint64_t len, uint64_t* out_bits,
                  uint32_t flags, void* stream);

/*
 * Per-read query of a device batch of n_reads equal-length DNA reads
 * ([cuSBF] §IV-E, Algorithm 2, on the read sets of §V-A; the page queries
 * records joined by an invalid separator, §IV-F, and so spends work on the
 * k-1 starts per record that straddle two records; here no read's work
 * crosses into the next).  Read r is the read_len bytes at
 * d_reads + r * stride (stride >= read_len when n_reads > 1, at most 2^25;
 * the bytes between reads never enter an answer).  Each read has
 * nkr = read_len - k + 1 k-mers and gets rch = ceil(nkr / 32) uint32_t words
 * of d_out (device, n_reads * rch words, fully overwritten): read r's k-mer
 * 32j + i is bit i of word rch * r + j, 1 iff present (every s-mer hits, as
 * in sbf_query_seq); k-mers with a non-ACGT base answer 0, and so do the bits
 * past nkr.  The answers equal sbf_query_seq's bits r * stride + i of the
 * batch queried as one sequence, for i < nkr.  Asynchronous on `stream`.  A
 * DNA filter whose query takes 32 k-mers per lane (as in sbf_query_seq) runs
 * a per-read kernel with no staging; any other DNA filter queries the batch
 * as one sequence into a handle-owned answer buffer (grown on demand, which
 * synchronizes `stream`) and cuts the reads' words out of it.  n_reads = 0 or
 * read_len < k is a no-op.  Errors: SBF_EINVAL (NULL handle or pointer,
 * stride < read_len, stride > 2^25, n_reads * rch >= 2^32), SBF_EUNSUPPORTED
 * (protein and triplet filters), SBF_ENOMEM, SBF_EDEVICE.
 */
int sbf_query_reads(sbf_t* h, const char* d_reads, uint64_t n_reads, uint32_t read_len,
                    uint64_t stride, uint32_t* d_out, void* stream);

/*
 * Chunk size of the host pipeline ([cuSBF] §IV-G host staging; the page gives
 * no chunk size), in k-mer starts (rounded up to a multiple
 * of 64; 64 <= chunk_bases <= 2^34; default 2^26).  Each of the three slots
 * holds chunk_bases + 64 bytes of pinned input, the same on the device, its
 * packed form and chunk_bases/64 + 1 answer words (pinned and device).
 * Buffers of another size are freed; the next host call allocates anew.
 */
int sbf_set_staging(sbf_t* h, uint64_t chunk_bases);

/* ---- FASTA / FASTQ input ([cuSBF] §IV-A input forms, §IV-F, §IV-G) -------
 * A FASTA or FASTQ file, plain or gzip-compressed (detected from the data),
 * becomes the "normalized stream": the sequence of each record with line
 * breaks and other bytes <= 0x20 removed, records joined by one 'N', so every
 * k-mer that spans two records is invalid ([cuSBF] §IV-F).  FASTA: '>' starts
 * a record, ';' lines are comments.  FASTQ: '@' header, sequence lines up to a
 * '+' line, then quality lines until they hold as many bytes as the sequence.
 * Record r spans [start_r, end_r) of the stream, start_0 = 0 and
 * start_r = end_{r-1} + 1.
 */
typedef struct sbf_fastx sbf_fastx_t;

/* Open a reader (host only, no device use).  SBF_EIO if the file cannot be
 * opened. */
int sbf_fastx_open(sbf_fastx_t** out, const char* path);

/*
 * Next piece of the normalized stream: up to cap bytes into buf, *len bytes
 * written.  If ends is not NULL, the stream offsets end_r of the records that
 * end within this piece go to ends[0 .. *n_ends) (the call stops early rather
 * than drop one when ends_cap are reported).  *len == 0 and *n_ends == 0
 * together mean the end of the stream.  SBF_EIO on a read error or malformed
 * input (text in sbf_last_error); the reader is then unusable.
 */
int sbf_fastx_read(sbf_fastx_t* r, char* buf, uint64_t cap, uint64_t* len,
                   uint64_t* ends, uint64_t ends_cap, uint64_t* n_ends);

/* Records started so far (0 for NULL).  Reader bookkeeping, not defined by
 * the page. */
uint64_t sbf_fastx_records(const sbf_fastx_t* r);

/* Close a reader and free its buffers; NULL is a no-op (not defined by the
 * page). */
int sbf_fastx_close(sbf_fastx_t* r);

typedef struct sbf_fastx_stats {
    uint64_t records;     /* records in the file */
    uint64_t bases;       /* length of the normalized stream, separators included */
    uint64_t chunks;      /* pipeline chunks processed */
    double parse_seconds; /* host time spent reading, decompressing and normalizing */
    double total_seconds; /* wall time of the call */
} sbf_fastx_stats_t;

/*
 * Insert every valid k-mer of a FASTA/FASTQ file through the host pipeline
 * (DNA filters; SBF_EUNSUPPORTED for protein and triplet filters, whose
 * alphabets the 'N' record separator does not fit):
 * the reader writes the normalized stream straight into the pinned chunk
 * buffers while the device works on the previous chunk.  Synchronizes.
 * stats may be NULL.  SBF_EIO for file errors; no partial insert is undone.
 */
int sbf_insert_fastx(sbf_t* h, const char* path, sbf_fastx_stats_t* stats);

/*
 * Query a FASTA/FASTQ file: for record r < cap, hits[r] = number of its
 * k-mers reported present and kmers[r] = number of its k-mer starts
 * (max(0, length - k + 1)); either array may be NULL.  Records beyond cap are
 * processed but not reported; stats->records gives their number.
 * Synchronizes.
 */
int sbf_query_fastx(sbf_t* h, const char* path, uint64_t* hits, uint64_t* kmers, uint64_t cap,
                    sbf_fastx_stats_t* stats);

/*
 * Allocation-free insert of a device sequence, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same result as sbf_insert_seq with
 * SBF_DEVICE, asynchronous on `stream`, but the packed codes and validity go
 * to a static device array of the library (24 MiB per device, held until the
 * process ends) instead of the handle's staging buffers, and the call makes
 * no allocation of any kind.  DNA filters: len <= 2^26 bases, larger len is
 * SBF_EINVAL (split the input into pieces overlapping by k-1 bases); protein
 * and triplet filters read the text directly and take any length.
 * All calls on one device share that array: two calls that may overlap on
 * one device (other streams, other handles, other threads) race and must be
 * serialized by the caller.  len < k is a no-op.  Errors: SBF_EINVAL (NULL
 * handle or sequence, len over the limit), SBF_EDEVICE.
 */
int sbf_insert_seq_noalloc(sbf_t* h, const char* d_seq, uint64_t len, void* stream);

/*
 * False-positive probe ([cuSBF] §V-D): query n k-mers drawn on the device
 * from the SplitMix64 stream seeded with `seed` (k-mer i = output i shifted
 * right by 64-2k) and store the number of positives in *hits (host).
 * Synchronizes.
 */
int sbf_fpr_probe(sbf_t* h, uint64_t n, uint64_t seed, uint64_t* hits);

/* As sbf_fpr_probe, asynchronous: the count lands in *d_hits (device). */
int sbf_fpr_probe_device(sbf_t* h, uint64_t n, uint64_t seed, uint64_t* d_hits, void* stream);

/* ---- measurement support (not the method) ------------------------------
 * Matched memory ceilings for the filter kernels' access patterns ([cuSBF]
 * §V-E speed of light): n operations on uniformly random shards of a device
 * table of nshard 32-byte shards (uint64_t[4 * nshard], nshard a power of
 * two; shard of operation j = SplitMix64 output j + 1 of the seed, masked).
 * Asynchronous on `stream`; the caller times them.  SBF_EINVAL for NULL
 * pointers or an nshard that is not a power of two; n must be below 2^60.
 */

/* Read the 32 bytes of each operation's shard (two 16-byte loads per lane),
 * as the query and probe kernels read theirs.  d_sink (one device word) is
 * written only if the XOR of everything read hits a fixed 64-bit value. */
int sbf_membench_shard_reads(const uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed,
                             uint64_t* d_sink, void* stream);

/* OR one bit into each of the four words of each operation's shard, four
 * adjacent lanes with one 64-bit atomic each, as the insert flushes a run's
 * record.  Modifies the table. */
int sbf_membench_shard_ors(uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed, void* stream);

/* Random 32-byte OR-updates of each operation's shard, four adjacent lanes
 * with one 64-bit update each, in the form `mode` selects: bits 0-1 = 0 a
 * device-scope atomic OR (as sbf_membench_shard_ors), 1 a workgroup-scope
 * atomic OR, 2 a plain load, OR and store (not atomic: concurrent updates of
 * one word can be lost; it measures a rate, not a filter); bit 2 confines the
 * shards of workgroup b to the eighth of the table numbered b mod 8 (needs
 * nshard >= 8).  Modifies the table.  SBF_EINVAL for other modes. */
int sbf_membench_shard_rmw(uint64_t* d_table, uint64_t nshard, uint64_t n, uint64_t seed, uint32_t mode,
                           void* stream);

/* VALU issue rate: 8192 workgroups of 256 lanes, each lane running `iters`
 * rounds of eight independent instructions of one form (kind 0: v_xor_b32 on
 * VGPRs, the two-operand 32-bit logic/add/shift forms; kind 1:
 * v_mad_u64_u32, a 64-bit form), i.e. 8192 * 256 * 8 * iters lane-
 * instructions.  Registers only; d_sink (one device word) is written only if
 * the results hit a fixed value.  Asynchronous on `stream`; the caller times
 * it.  SBF_EINVAL for a NULL d_sink, kind > 1 or iters outside 1 .. 2^32. */
int sbf_membench_valu(uint32_t kind, uint64_t iters, uint64_t* d_sink, void* stream);

/* Static text for a return code (error reporting is this library's; the page
 * states none). */
const char* sbf_strerror(int code);

/* Text of the calling thread's last error ("" if none); valid until the
 * thread's next call into the library. */
const char* sbf_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SBF_H */
