// sbf_internal.hpp -- host-side types shared by the library's translation
// units: launch arguments, kernel sets and the specialization registry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbf {

// Arguments of one insert or query launch over a packed sequence.
struct SeqArgs {
    const uint32_t* codes;  // packed bases, 16 per word
    const uint32_t* valid;  // validity bits, 32 per word
    uint64_t ncw;           // code words
    uint64_t nvw;           // validity words
    uint64_t nk;            // k-mer starts: len - k + 1
    uint64_t* filter;       // uint64_t[4N]
    uint32_t shard_mask;    // N - 1
    uint64_t* out;          // query bits (query only)
    hipStream_t stream;
    // Protein and triplet alphabets read the ASCII text itself: symbol j is
    // byte j (protein) or bytes 3j..3j+2 (triplet); nk counts symbol starts.
    // So does a DNA query through KernelSet::query_text (base j = byte j).
    const char* text;
    uint64_t nsym;
    // Per-read DNA query (KernelSet::query_reads): read r is the rlen bytes
    // at text + r * stride, nsym the bytes from text to the last read's end,
    // nk the batch's chunks (rchunks = ceil((rlen - k + 1) / 32) per read),
    // out the answer words (uint32_t[nk]).
    uint64_t stride;
    uint32_t rlen;
    uint32_t rchunks;
};

// Arguments of one false-positive probe launch.
struct ProbeArgs {
    const uint64_t* filter;
    uint32_t shard_mask;
    uint64_t n;
    uint64_t seed;
    unsigned long long* hits;  // device counter, accumulated into
    hipStream_t stream;
};

// Runtime parameters, used by the generic (non-specialized) kernels.
struct Params {
    uint32_t kind, k, m, s, H;
    uint32_t alpha;  // SBF_ALPHABET_*: 0 DNA, 1 protein, 2 DNA triplets
};

typedef hipError_t (*SeqLaunch)(const SeqArgs&, const Params&);
typedef hipError_t (*ProbeLaunch)(const ProbeArgs&, const Params&);

struct KernelSet {
    SeqLaunch insert;
    SeqLaunch query;
    ProbeLaunch probe;
    int specialized;
    // DNA query straight from ASCII (SeqArgs.text, nsym = bytes), or null:
    // the sequence is then packed first and `query` reads the codes
    SeqLaunch query_text = nullptr;
    // DNA insert straight from ASCII (SeqArgs.text, nsym = bytes), or null
    SeqLaunch insert_text = nullptr;
    // Per-read DNA query of a batch of equal-length reads (SeqArgs.stride,
    // rlen, rchunks), or null: sbf_query_reads then queries the batch as one
    // sequence and cuts each read's answers out of it
    SeqLaunch query_reads = nullptr;
};

// One row of a specialization table (see sbf_spec_list.hpp).
struct SpecEntry {
    uint32_t kind, k, m, s, H;
    KernelSet (*make)();
};

// Compile-time specialized kernel sets; false if (kind,k,m,s,H) has none.
bool find_specialized(const Params& p, KernelSet* out);
// Kernel set for any valid parameters (one k-mer per lane, runtime loops).
KernelSet generic_kernels();
// Kernel set of the protein (alpha 1) or triplet (alpha 2) Super Bloom
// filter: compile-time specialized for a few parameter sets, else run-time.
KernelSet alpha_kernels(const Params& P);

// Small utility launches.
hipError_t launch_pack(const char* ascii, uint64_t len, uint32_t* codes, uint32_t* valid, hipStream_t st);
hipError_t launch_fill_zero(uint64_t* p, uint64_t nwords, hipStream_t st);
// Answers of a batch of n equal-length reads (read r at byte r * stride,
// nkr = len - k + 1 k-mers each) cut out of the answers of the batch queried
// as one sequence (bits: one bit per k-mer start, nbw words): read r gets
// words rch * r .. rch * r + rch - 1 of out, k-mer 32j + i at bit i of word
// j, 0 past its last k-mer.
hipError_t launch_reads_remap(const uint64_t* bits, uint64_t nbw, uint64_t n, uint64_t stride, uint32_t nkr,
                              uint32_t rch, uint32_t* out, hipStream_t st);

}  // namespace sbf
