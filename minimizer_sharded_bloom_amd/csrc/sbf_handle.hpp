// sbf_handle.hpp -- the filter handle behind sbf_t, shared by the C-ABI
// translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sbf.h"
#include "sbf_internal.hpp"

namespace sbf {

// Staging of host-resident sequences ([cuSBF] §IV-G host staging): a ring
// of kHostSlots slots; slot b holds a pinned input chunk, its device copy,
// packed codes and validity, and the chunk's answer words (device and
// pinned), and runs on its own stream, so the host fills one slot while the
// copies and kernels of the others run.  Created on first use and kept until
// the handle is destroyed.
constexpr int kHostSlots = 3;

struct HostStaging {
    uint64_t chunk = 1ull << 26;  // k-mer starts per chunk, a multiple of 64
    uint64_t built_for = 0;       // chunk size the buffers below were sized for
    hipStream_t s[kHostSlots] = {};
    hipEvent_t done[kHostSlots] = {};  // slot's copy, kernels and answer copy finished
    char* h_in[kHostSlots] = {};       // pinned
    uint64_t* h_out[kHostSlots] = {};  // pinned
    char* d_in[kHostSlots] = {};
    uint32_t* d_codes[kHostSlots] = {};
    uint32_t* d_valid[kHostSlots] = {};
    uint64_t* d_out[kHostSlots] = {};
};

}  // namespace sbf

struct sbf_handle {
    sbf::Params P;
    uint64_t num_shards;
    uint32_t wps;  // 64-bit words per shard: 4, or 8 for the wide-block variant
    uint64_t* d_filter;
    sbf::KernelSet ks;
    int device;
    // packing of device-resident sequences (SBF_DEVICE calls)
    uint32_t* d_codes;
    uint32_t* d_valid;
    uint64_t packed_cap;  // bases
    // answers of a read batch queried as one sequence (sbf_query_reads
    // without a per-read kernel)
    uint64_t* d_rbits;
    uint64_t rbits_cap;  // words
    unsigned long long* d_hits;
    sbf::HostStaging host;
};

namespace sbf {
// Error reporting shared by the C-ABI translation units (sbf_api.cpp).
int fail(int code, const char* what);
int fail_hip(hipError_t e, const char* what);
void ok();
int set_device(const sbf_t* h);
SeqArgs seq_args(sbf_t* h, const uint32_t* codes, const uint32_t* valid, uint64_t len, uint64_t* out,
                 hipStream_t st);
// Protein and triplet filters: bytes per symbol (1 or 3), symbols in len
// bytes, and launch arguments over the text itself.
uint32_t symbol_bytes(const sbf_t* h);
uint64_t symbols_of(const sbf_t* h, uint64_t len);
SeqArgs text_args(sbf_t* h, const char* text, uint64_t len, uint64_t* out, hipStream_t st);
void free_host_staging(HostStaging& hs);
// Host-resident insert / query through the chunked pipeline (sbf_host.cpp);
// both synchronize before returning.
int host_insert(sbf_t* h, const char* seq, uint64_t len, hipStream_t st);
int host_query(sbf_t* h, const char* seq, uint64_t len, uint64_t* out_bits, hipStream_t st);
}  // namespace sbf
