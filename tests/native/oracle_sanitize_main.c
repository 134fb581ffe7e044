/* Driver that runs the CPU oracle (oracle/sbf_oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer: every filter kind and alphabet, inputs of
 * edge lengths with invalid bytes, single- and multi-threaded insert and
 * query, sampled drivers, positions and the probe.  It also checks the Bloom
 * property of the method (every valid inserted k-mer queries present) on the
 * single-threaded insert, and that the threaded insert and query give the
 * same words and answers.
 * Exit status 0 = no sanitizer report and no failed check. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/sbf_oracle.h"

static uint64_t rng_state = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* len bytes over `alphabet`, with about one byte in 64 replaced by `bad` */
static char* make_text(uint64_t len, const char* alphabet, char bad)
{
    char* t = malloc(len ? len : 1);
    size_t na = strlen(alphabet);
    for (uint64_t i = 0; i < len; ++i) {
        uint64_t r = next_u64();
        t[i] = (r & 63) == 0 ? bad : alphabet[(r >> 8) % na];
    }
    return t;
}

static int failures = 0;

static void run_case(int kind, unsigned alpha, unsigned k, unsigned m, unsigned s, unsigned H, uint64_t bits,
                     uint64_t len)
{
    const char* al = alpha == OSBF_ALPHA_PROTEIN ? "ACDEFGHIKLMNPQRSTVWYacdwy" : "ACGTacgt";
    char bad = alpha == OSBF_ALPHA_PROTEIN ? '*' : 'N';
    unsigned sb = alpha == OSBF_ALPHA_TRIPLET ? 3 : 1;
    osbf* f = osbf_create_alpha(kind, alpha, k, m, s, H, bits);
    if (!f) {
        fprintf(stderr, "create failed: kind %d alpha %u (%u,%u,%u,%u)\n", kind, alpha, k, m, s, H);
        ++failures;
        return;
    }
    osbf* g = osbf_create_alpha(kind, alpha, k, m, s, H, bits);
    char* text = make_text(len, al, bad);
    osbf_insert_seq(f, text, len);
    osbf_insert_seq_mt(g, text, len, 3);
    /* the threaded insert spells the per-k-mer definition out again: the
     * two filters must agree word for word */
    const uint64_t nwords = osbf_num_shards(f) * osbf_words_per_shard(f);
    if (memcmp(osbf_words(f), osbf_words(g), nwords * 8) != 0) {
        fprintf(stderr, "threaded insert differs: kind %d alpha %u len %llu\n", kind, alpha, (unsigned long long)len);
        ++failures;
    }
    uint64_t nsym = len / sb;
    uint64_t nk = nsym >= k ? nsym - k + 1 : 0;
    uint64_t nw = (nk + 63) / 64 + 1;
    uint64_t* out = calloc(nw, 8);
    uint64_t* out2 = calloc(nw, 8);
    uint64_t* chk = calloc(nw, 8);
    osbf_query_seq(f, text, len, out);
    osbf_query_seq_mt(f, text, len, out2, 4);
    if (nw && memcmp(out, out2, nw * 8) != 0) {
        fprintf(stderr, "threaded query differs: kind %d alpha %u len %llu\n", kind, alpha, (unsigned long long)len);
        ++failures;
    }
    /* every valid inserted k-mer is present (checked on lightly loaded
     * filters, where a missing bit is not hidden by saturation) */
    for (uint64_t p = 0; bits >= (1u << 16) && p < nk; ++p) {
        uint64_t x;
        /* the pack functions return 0 for a valid k-mer, -1 otherwise */
        int valid = (alpha == OSBF_ALPHA_DNA ? osbf_pack_kmer(text + p, k, &x)
                                             : osbf_pack_kmer_alpha(alpha, text, p, k, &x)) == 0;
        if (valid && !((out[p >> 6] >> (p & 63)) & 1)) {
            fprintf(stderr, "false negative: kind %d alpha %u len %llu pos %llu\n", kind, alpha, (unsigned long long)len,
                    (unsigned long long)p);
            ++failures;
            break;
        }
    }
    if (nk) {
        uint64_t pos[5] = {0, nk - 1, nk / 2, nk / 3, nk > 1 ? 1 : 0};
        uint8_t ans[5];
        osbf_query_positions(f, text, len, pos, 5, ans);
    }
    if (alpha == OSBF_ALPHA_DNA) {
        osbf_insert_seq_sampled_mt(f, text, len, 7, 3, 2);
        osbf_query_seq_sampled_mt(f, text, len, out, chk, 7, 3, 2);
    }
    (void)osbf_fpr_probe(f, 2000, next_u64());
    osbf_destroy(g);
    free(out);
    free(out2);
    free(chk);
    free(text);
    osbf_destroy(f);
}

int main(void)
{
    static const uint64_t lens[] = {0, 1, 8, 30, 31, 32, 33, 63, 64, 65, 127, 1000, 4099};
    static const unsigned dna[][4] = {{31, 16, 28, 4}, {9, 5, 6, 3}, {32, 16, 28, 4}, {31, 31, 31, 12}, {5, 3, 4, 2},
                                      {1, 1, 1, 1}};
    for (unsigned c = 0; c < sizeof(dna) / sizeof(dna[0]); ++c)
        for (unsigned i = 0; i < sizeof(lens) / sizeof(lens[0]); ++i)
            for (int kind = OSBF_KIND_SBF; kind <= OSBF_KIND_WIDE; ++kind)
                for (int big = 0; big < 2; ++big)
                    run_case(kind, OSBF_ALPHA_DNA, dna[c][0], dna[c][1], dna[c][2], dna[c][3],
                             big ? 1u << 20 : 1u << (7 + c), lens[i]);
    static const unsigned prot[][4] = {{12, 6, 10, 4}, {9, 4, 7, 3}, {1, 1, 1, 2}};
    static const unsigned trip[][4] = {{10, 5, 8, 4}, {7, 3, 7, 2}, {1, 1, 1, 4}};
    for (unsigned c = 0; c < 3; ++c)
        for (unsigned i = 0; i < sizeof(lens) / sizeof(lens[0]); ++i) {
            for (int big = 0; big < 2; ++big) {
                const uint64_t bits = big ? 1u << 20 : 4096;
                run_case(OSBF_KIND_SBF, OSBF_ALPHA_PROTEIN, prot[c][0], prot[c][1], prot[c][2], prot[c][3], bits, lens[i]);
                run_case(OSBF_KIND_SBF, OSBF_ALPHA_TRIPLET, trip[c][0], trip[c][1], trip[c][2], trip[c][3], bits,
                         3 * lens[i] + (lens[i] % 3));
            }
        }
    printf("oracle sanitizer run: %d failures\n", failures);
    return failures ? 1 : 0;
}
