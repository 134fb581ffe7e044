// sbf_api.cpp -- the extern "C" surface of libsbf.so (declared in
// include/sbf.h): argument checks, filter ownership, staging buffers and
// dispatch to the specialized or generic kernel sets.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/sbf.h"
#include "sbf_handle.hpp"

namespace sbf {
const SpecEntry* spec_table_m12(size_t* n);
const SpecEntry* spec_table_m16(size_t* n);
const SpecEntry* spec_table_m20(size_t* n);
const SpecEntry* spec_table_extra(size_t* n);
const SpecEntry* spec_table_slice_s_a(size_t* n);
const SpecEntry* spec_table_slice_s_b(size_t* n);
const SpecEntry* spec_table_slice_m_a(size_t* n);
const SpecEntry* spec_table_slice_m_b(size_t* n);
const SpecEntry* spec_table_slice_m_c(size_t* n);
const SpecEntry* spec_table_slice_h(size_t* n);
const SpecEntry* spec_table_wide(size_t* n);
const SpecEntry* spec_table_grid_best_a(size_t* n);
const SpecEntry* spec_table_grid_best_b(size_t* n);

bool find_specialized(const Params& p, KernelSet* out)
{
    if (p.alpha != SBF_ALPHABET_DNA)
        return false;
    typedef const SpecEntry* (*TableFn)(size_t*);
    static const TableFn tables[] = {spec_table_m12,       spec_table_m16,       spec_table_m20,
                                     spec_table_extra,     spec_table_slice_s_a, spec_table_slice_s_b,
                                     spec_table_slice_m_a, spec_table_slice_m_b, spec_table_slice_m_c,
                                     spec_table_slice_h,   spec_table_wide,      spec_table_grid_best_a,
                                     spec_table_grid_best_b};
    for (TableFn fn : tables) {
        size_t n = 0;
        const SpecEntry* t = fn(&n);
        for (size_t i = 0; i < n; ++i) {
            if (t[i].kind == p.kind && t[i].k == p.k && t[i].m == p.m && t[i].s == p.s && t[i].H == p.H) {
                *out = t[i].make();
                return true;
            }
        }
    }
    return false;
}
}  // namespace sbf

namespace {
thread_local std::string g_last_error;

// Packed staging of sbf_insert_seq_noalloc, for callers that cannot allocate:
// the code words of up to kNoAllocMaxBases bases, then their validity words
// (24 MiB).  Each device the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never a
// device address: kernels get the address that hipGetSymbolAddress returns
// for the current device (noalloc_scratch below).
constexpr uint64_t kNoAllocMaxBases = 1ull << 26;
constexpr uint64_t kNoAllocCodeWords = kNoAllocMaxBases / 16;   // 16 bases per code word
constexpr uint64_t kNoAllocValidWords = kNoAllocMaxBases / 32;  // 32 bases per validity word

// sbf_query_reads: the per-read kernel addresses a wave's bytes with 32-bit
// offsets from its first read, at most 65 strides away
constexpr uint64_t kReadsMaxStride = 1ull << 25;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until resolved
}  // namespace

static __device__ __align__(256) uint32_t scratch[kNoAllocCodeWords + kNoAllocValidWords];

namespace sbf {

int fail(int code, const char* what)
{
    g_last_error = what;
    return code;
}

// A HIP call that fails also leaves its error as the thread's last HIP
// error, which the launch checks (hipGetLastError after a launch) would
// report again on a later, unrelated call.  The error is recorded here and
// then cleared.
int fail_hip(hipError_t e, const char* what)
{
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? SBF_ENOMEM : SBF_EDEVICE;
}

void ok() { g_last_error.clear(); }

// Every entry point that launches work comes through here first: an error
// left behind by an earlier HIP call of the caller's is not this call's, so
// it is dropped before the call's own launches are checked.
int set_device(const sbf_t* h)
{
    (void)hipGetLastError();
    hipError_t e = hipSetDevice(h->device);
    return e == hipSuccess ? SBF_OK : fail_hip(e, "hipSetDevice");
}

// Device address of `device`'s copy of the static scratch array, resolved
// once per device with that device current (it must be current here).  Called
// when a filter is created on the device, and again by the allocation-free
// entry point if that did not succeed.
int noalloc_scratch(int device, uint32_t** out)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(SBF_EDEVICE, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return fail_hip(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[device] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[device];
    return SBF_OK;
}

uint64_t code_words(uint64_t len) { return (len + 15) / 16; }
uint64_t valid_words(uint64_t len) { return (len + 31) / 32; }

SeqArgs seq_args(sbf_t* h, const uint32_t* codes, const uint32_t* valid, uint64_t len, uint64_t* out,
                 hipStream_t st)
{
    SeqArgs a{};
    a.codes = codes;
    a.valid = valid;
    a.ncw = code_words(len);
    a.nvw = valid_words(len);
    a.nk = len - h->P.k + 1;
    a.filter = h->d_filter;
    a.shard_mask = (uint32_t)(h->num_shards - 1);
    a.out = out;
    a.stream = st;
    return a;
}

uint32_t symbol_bytes(const sbf_t* h) { return h->P.alpha == SBF_ALPHABET_TRIPLET ? 3u : 1u; }

uint64_t symbols_of(const sbf_t* h, uint64_t len) { return len / symbol_bytes(h); }

SeqArgs text_args(sbf_t* h, const char* text, uint64_t len, uint64_t* out, hipStream_t st)
{
    SeqArgs a{};
    a.text = text;
    a.nsym = symbols_of(h, len);
    a.nk = a.nsym - h->P.k + 1;
    a.filter = h->d_filter;
    a.shard_mask = (uint32_t)(h->num_shards - 1);
    a.out = out;
    a.stream = st;
    return a;
}

}  // namespace sbf

namespace {
using namespace sbf;

int create_impl(sbf_t** out, const sbf::Params& P, uint64_t bits)
{
    if (!out)
        return fail(SBF_EINVAL, "out is NULL");
    if (P.alpha > SBF_ALPHABET_TRIPLET)
        return fail(SBF_EINVAL, "unknown alphabet");
    if (P.alpha == SBF_ALPHABET_PROTEIN && (P.k < 1 || P.k > 12))
        return fail(SBF_EINVAL, "k must be in 1..12 for proteins (5 bits per symbol)");
    if (P.alpha == SBF_ALPHABET_TRIPLET && (P.k < 1 || P.k > 10))
        return fail(SBF_EINVAL, "k must be in 1..10 for triplets (6 bits per symbol)");
    if (P.k < 1 || P.k > 32)
        return fail(SBF_EINVAL, "k must be in 1..32");
    if (P.kind != SBF_KIND_BBF && (P.m < 1 || P.m > P.k))
        return fail(SBF_EINVAL, "m must be in 1..k");
    if (P.kind != SBF_KIND_BBF && (P.s < 1 || P.s > P.k))
        return fail(SBF_EINVAL, "s must be in 1..k");
    if (P.H < 1 || P.H > 64)
        return fail(SBF_EINVAL, "H must be in 1..64");
    if (bits < 1 || bits > (1ull << 40))
        return fail(SBF_EINVAL, "bits must be in 1..2^40");
    const uint32_t wps = P.kind == SBF_KIND_WIDE ? 8u : 4u;
    const uint64_t block = 64ull * wps;
    const uint64_t need = (bits + block - 1) / block;
    uint64_t n = 1;
    while (n < need)
        n <<= 1;

    sbf_t* h = new (std::nothrow) sbf_t();
    if (!h)
        return fail(SBF_ENOMEM, "host allocation failed");
    h->P = P;
    h->num_shards = n;
    h->wps = wps;
    if (P.alpha != SBF_ALPHABET_DNA)
        h->ks = sbf::alpha_kernels(P);
    else if (!sbf::find_specialized(P, &h->ks))
        h->ks = sbf::generic_kernels();
    (void)hipGetLastError();  // an earlier call's error is not this one's (see set_device)
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "hipGetDevice");
    }
    e = hipMalloc(reinterpret_cast<void**>(&h->d_filter), 8ull * wps * n);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "hipMalloc(filter)");
    }
    e = hipMalloc(reinterpret_cast<void**>(&h->d_hits), sizeof(unsigned long long));
    if (e != hipSuccess) {
        (void)hipFree(h->d_filter);
        delete h;
        return fail_hip(e, "hipMalloc(counter)");
    }
    e = sbf::launch_fill_zero(h->d_filter, (uint64_t)wps * n, nullptr);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(h->d_filter);
        (void)hipFree(h->d_hits);
        delete h;
        return fail_hip(e, "zeroing the filter");
    }
    // set-up of the allocation-free insert on this device; a failure here
    // only matters to that entry point, which resolves again and reports it
    uint32_t* unused = nullptr;
    (void)sbf::noalloc_scratch(h->device, &unused);
    *out = h;
    ok();
    return SBF_OK;
}

int grow_packed(sbf_t* h, uint64_t len, hipStream_t st)
{
    if (h->packed_cap >= len)
        return SBF_OK;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return fail_hip(e, "staging");
    if (h->d_codes)
        (void)hipFree(h->d_codes);
    if (h->d_valid)
        (void)hipFree(h->d_valid);
    h->d_codes = nullptr;
    h->d_valid = nullptr;
    h->packed_cap = 0;
    const uint64_t n = len + len / 4 + 4096;
    e = hipMalloc(reinterpret_cast<void**>(&h->d_codes), 4 * code_words(n));
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void**>(&h->d_valid), 4 * valid_words(n));
    if (e != hipSuccess) {
        if (h->d_codes)
            (void)hipFree(h->d_codes);
        h->d_codes = nullptr;
        h->d_valid = nullptr;
        return fail_hip(e, "hipMalloc(packed staging)");
    }
    h->packed_cap = n;
    return SBF_OK;
}

// Answer words of a read batch queried as one sequence.
int grow_rbits(sbf_t* h, uint64_t words, hipStream_t st)
{
    if (h->rbits_cap >= words)
        return SBF_OK;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return fail_hip(e, "answer staging");
    if (h->d_rbits)
        (void)hipFree(h->d_rbits);
    h->d_rbits = nullptr;
    h->rbits_cap = 0;
    const uint64_t n = words + words / 4 + 64;
    e = hipMalloc(reinterpret_cast<void**>(&h->d_rbits), 8 * n);
    if (e != hipSuccess) {
        h->d_rbits = nullptr;
        return fail_hip(e, "hipMalloc(answer staging)");
    }
    h->rbits_cap = n;
    return SBF_OK;
}

// Pack a device-resident sequence into the handle's staging buffers.
int stage_packed(sbf_t* h, const char* d_seq, uint64_t len, hipStream_t st)
{
    int rc = grow_packed(h, len, st);
    if (rc)
        return rc;
    hipError_t e = sbf::launch_pack(d_seq, len, h->d_codes, h->d_valid, st);
    return e == hipSuccess ? SBF_OK : fail_hip(e, "pack launch");
}

int check_flags(uint32_t flags)
{
    return (flags == SBF_HOST || flags == SBF_DEVICE) ? SBF_OK : fail(SBF_EINVAL, "flags must be SBF_HOST or SBF_DEVICE");
}

}  // namespace

extern "C" {

int sbf_create(sbf_t** out, uint32_t k, uint32_t m, uint32_t s, uint32_t H, uint64_t bits)
{
    sbf::Params P{SBF_KIND_SBF, k, m, s, H};
    return create_impl(out, P, bits);
}

int sbf_create_bbf(sbf_t** out, uint32_t k, uint32_t H, uint64_t bits)
{
    sbf::Params P{SBF_KIND_BBF, k, 0, 0, H};
    return create_impl(out, P, bits);
}

int sbf_create_wide(sbf_t** out, uint32_t k, uint32_t m, uint32_t s, uint32_t H, uint64_t bits)
{
    sbf::Params P{SBF_KIND_WIDE, k, m, s, H};
    return create_impl(out, P, bits);
}

int sbf_create_alphabet(sbf_t** out, uint32_t alphabet, uint32_t k, uint32_t m, uint32_t s, uint32_t H,
                        uint64_t bits)
{
    sbf::Params P{SBF_KIND_SBF, k, m, s, H, alphabet};
    return create_impl(out, P, bits);
}

int sbf_destroy(sbf_t* h)
{
    if (!h)
        return SBF_OK;
    (void)hipSetDevice(h->device);
    hipError_t e = hipDeviceSynchronize();
    (void)hipFree(h->d_filter);
    (void)hipFree(h->d_hits);
    if (h->d_codes)
        (void)hipFree(h->d_codes);
    if (h->d_valid)
        (void)hipFree(h->d_valid);
    if (h->d_rbits)
        (void)hipFree(h->d_rbits);
    sbf::free_host_staging(h->host);
    delete h;
    if (e != hipSuccess)
        return fail_hip(e, "sbf_destroy");
    ok();
    return SBF_OK;
}

int sbf_clear(sbf_t* h, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipError_t e = sbf::launch_fill_zero(h->d_filter, (uint64_t)h->wps * h->num_shards, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail_hip(e, "clear launch");
    ok();
    return SBF_OK;
}

int sbf_info(const sbf_t* h, sbf_info_t* o)
{
    if (!h || !o)
        return fail(SBF_EINVAL, "NULL argument");
    o->k = h->P.k;
    o->m = h->P.m;
    o->s = h->P.s;
    o->H = h->P.H;
    o->kind = h->P.kind;
    o->specialized = (uint32_t)h->ks.specialized;
    o->num_shards = h->num_shards;
    o->filter_bytes = 8ull * h->wps * h->num_shards;
    o->words_per_shard = h->wps;
    o->alphabet = h->P.alpha;
    ok();
    return SBF_OK;
}

int sbf_copy_filter(const sbf_t* h, void* dst, uint64_t bytes, uint32_t flags, void* stream)
{
    if (!h || !dst)
        return fail(SBF_EINVAL, "NULL argument");
    if (check_flags(flags))
        return SBF_EINVAL;
    const uint64_t fbytes = 8ull * h->wps * h->num_shards;
    if (bytes < fbytes)
        return fail(SBF_EINVAL, "destination smaller than the filter");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (flags == SBF_HOST) {
        e = hipMemcpyAsync(dst, h->d_filter, fbytes, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess)
            e = hipStreamSynchronize(st);
    } else {
        e = hipMemcpyAsync(dst, h->d_filter, fbytes, hipMemcpyDeviceToDevice, st);
    }
    if (e != hipSuccess)
        return fail_hip(e, "copy filter");
    ok();
    return SBF_OK;
}

const uint64_t* sbf_filter_device_ptr(const sbf_t* h) { return h ? h->d_filter : nullptr; }

void sbf_packed_words(uint64_t len, uint64_t* cw, uint64_t* vw)
{
    if (cw)
        *cw = code_words(len);
    if (vw)
        *vw = valid_words(len);
}

int sbf_pack(const char* d_ascii, uint64_t len, uint32_t* d_codes, uint32_t* d_valid, void* stream)
{
    if (len == 0) {
        ok();
        return SBF_OK;
    }
    if (!d_ascii || !d_codes || !d_valid)
        return fail(SBF_EINVAL, "NULL argument");
    (void)hipGetLastError();  // an earlier call's error is not this one's (see set_device)
    hipError_t e = sbf::launch_pack(d_ascii, len, d_codes, d_valid, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail_hip(e, "pack launch");
    ok();
    return SBF_OK;
}

int sbf_insert_packed(sbf_t* h, const uint32_t* d_codes, const uint32_t* d_valid, uint64_t len, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (h->P.alpha != SBF_ALPHABET_DNA)
        return fail(SBF_EUNSUPPORTED, "packed input is DNA only");
    if (len < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!d_codes || !d_valid)
        return fail(SBF_EINVAL, "NULL argument");
    int rc = set_device(h);
    if (rc)
        return rc;
    const sbf::SeqArgs a = seq_args(h, d_codes, d_valid, len, nullptr, (hipStream_t)stream);
    hipError_t e = h->ks.insert(a, h->P);
    if (e != hipSuccess)
        return fail_hip(e, "insert launch");
    ok();
    return SBF_OK;
}

int sbf_query_packed(sbf_t* h, const uint32_t* d_codes, const uint32_t* d_valid, uint64_t len, uint64_t* d_out,
                     void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (h->P.alpha != SBF_ALPHABET_DNA)
        return fail(SBF_EUNSUPPORTED, "packed input is DNA only");
    if (len < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!d_codes || !d_valid || !d_out)
        return fail(SBF_EINVAL, "NULL argument");
    int rc = set_device(h);
    if (rc)
        return rc;
    const sbf::SeqArgs a = seq_args(h, d_codes, d_valid, len, d_out, (hipStream_t)stream);
    hipError_t e = h->ks.query(a, h->P);
    if (e != hipSuccess)
        return fail_hip(e, "query launch");
    ok();
    return SBF_OK;
}

int sbf_insert_seq(sbf_t* h, const char* seq, uint64_t len, uint32_t flags, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (check_flags(flags))
        return SBF_EINVAL;
    if (symbols_of(h, len) < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!seq)
        return fail(SBF_EINVAL, "seq is NULL");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (flags == SBF_HOST)
        return sbf::host_insert(h, seq, len, st);
    if (h->P.alpha != SBF_ALPHABET_DNA) {
        hipError_t e = h->ks.insert(text_args(h, seq, len, nullptr, st), h->P);
        if (e != hipSuccess)
            return fail_hip(e, "insert");
        ok();
        return SBF_OK;
    }
    if (h->ks.insert_text && ((uintptr_t)seq & 15u) == 0) {
        // the insert kernel reads the ASCII itself (16-byte loads per lane)
        hipError_t e = h->ks.insert_text(text_args(h, seq, len, nullptr, st), h->P);
        if (e != hipSuccess)
            return fail_hip(e, "insert");
        ok();
        return SBF_OK;
    }
    rc = stage_packed(h, seq, len, st);
    if (rc)
        return rc;
    const sbf::SeqArgs a = seq_args(h, h->d_codes, h->d_valid, len, nullptr, st);
    hipError_t e = h->ks.insert(a, h->P);
    if (e != hipSuccess)
        return fail_hip(e, "insert");
    ok();
    return SBF_OK;
}

int sbf_query_seq(sbf_t* h, const char* seq, uint64_t len, uint64_t* out_bits, uint32_t flags, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (check_flags(flags))
        return SBF_EINVAL;
    if (symbols_of(h, len) < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!seq || !out_bits)
        return fail(SBF_EINVAL, "NULL argument");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (flags == SBF_HOST)
        return sbf::host_query(h, seq, len, out_bits, st);
    if (h->P.alpha != SBF_ALPHABET_DNA) {
        hipError_t e = h->ks.query(text_args(h, seq, len, out_bits, st), h->P);
        if (e != hipSuccess)
            return fail_hip(e, "query");
        ok();
        return SBF_OK;
    }
    if (h->ks.query_text && ((uintptr_t)seq & 15u) == 0) {
        // the query kernel reads the ASCII itself (16-byte loads per lane)
        hipError_t e = h->ks.query_text(text_args(h, seq, len, out_bits, st), h->P);
        if (e != hipSuccess)
            return fail_hip(e, "query");
        ok();
        return SBF_OK;
    }
    rc = stage_packed(h, seq, len, st);
    if (rc)
        return rc;
    const sbf::SeqArgs a = seq_args(h, h->d_codes, h->d_valid, len, out_bits, st);
    hipError_t e = h->ks.query(a, h->P);
    if (e != hipSuccess)
        return fail_hip(e, "query");
    ok();
    return SBF_OK;
}

int sbf_query_reads(sbf_t* h, const char* d_reads, uint64_t n_reads, uint32_t read_len, uint64_t stride,
                    uint32_t* d_out, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (h->P.alpha != SBF_ALPHABET_DNA)
        return fail(SBF_EUNSUPPORTED, "sbf_query_reads: DNA filters only (query protein or triplet text with sbf_query_seq)");
    if (n_reads == 0 || read_len < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!d_reads || !d_out)
        return fail(SBF_EINVAL, "NULL argument");
    if (n_reads > 1 && stride < read_len)
        return fail(SBF_EINVAL, "sbf_query_reads: stride is less than read_len");
    if (stride > kReadsMaxStride)
        return fail(SBF_EINVAL, "sbf_query_reads: stride exceeds 2^25 bytes");
    const uint32_t nkr = read_len - h->P.k + 1;  // k-mers per read
    const uint32_t rch = (nkr + 31) / 32;        // answer words per read
    if (n_reads > 0xFFFFFFFFull / rch)
        return fail(SBF_EINVAL, "sbf_query_reads: the batch has 2^32 or more answer words; split it");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    const uint64_t nbytes = (n_reads - 1) * stride + read_len;
    hipError_t e;
    if (h->ks.query_reads) {
        sbf::SeqArgs a = text_args(h, d_reads, nbytes, reinterpret_cast<uint64_t*>(d_out), st);
        a.nk = n_reads * rch;
        a.stride = stride;
        a.rlen = read_len;
        a.rchunks = rch;
        e = h->ks.query_reads(a, h->P);
    } else {
        // the batch as one sequence, then each read's answers cut out of it
        const uint64_t nbw = (nbytes - h->P.k + 1 + 63) / 64;
        rc = grow_rbits(h, nbw, st);
        if (rc)
            return rc;
        rc = sbf_query_seq(h, d_reads, nbytes, h->d_rbits, SBF_DEVICE, stream);
        if (rc)
            return rc;
        e = sbf::launch_reads_remap(h->d_rbits, nbw, n_reads, stride, nkr, rch, d_out, st);
    }
    if (e != hipSuccess)
        return fail_hip(e, "query_reads");
    ok();
    return SBF_OK;
}

int sbf_insert_seq_noalloc(sbf_t* h, const char* d_seq, uint64_t len, void* stream)
{
    if (!h)
        return fail(SBF_EINVAL, "handle is NULL");
    if (symbols_of(h, len) < h->P.k) {
        ok();
        return SBF_OK;
    }
    if (!d_seq)
        return fail(SBF_EINVAL, "seq is NULL");
    if (h->P.alpha == SBF_ALPHABET_DNA && len > kNoAllocMaxBases)
        return fail(SBF_EINVAL, "sbf_insert_seq_noalloc: len exceeds 2^26 bases, the size of its static staging");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (h->P.alpha != SBF_ALPHABET_DNA) {
        // protein and triplet kernels read the text itself: no staging
        e = h->ks.insert(text_args(h, d_seq, len, nullptr, st), h->P);
    } else {
        uint32_t* base = nullptr;
        rc = noalloc_scratch(h->device, &base);
        if (rc)
            return rc;
        // The pack writes every code and validity word that the insert reads
        // (its buffer ranges end at ceil(len/16) and ceil(len/32) words), so
        // nothing left by an earlier call needs clearing.
        uint32_t* codes = base;
        uint32_t* valid = base + kNoAllocCodeWords;
        e = sbf::launch_pack(d_seq, len, codes, valid, st);
        if (e == hipSuccess)
            e = h->ks.insert(seq_args(h, codes, valid, len, nullptr, st), h->P);
    }
    if (e != hipSuccess)
        return fail_hip(e, "insert");
    ok();
    return SBF_OK;
}

int sbf_fpr_probe_device(sbf_t* h, uint64_t n, uint64_t seed, uint64_t* d_hits, void* stream)
{
    if (!h || !d_hits)
        return fail(SBF_EINVAL, "NULL argument");
    int rc = set_device(h);
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = sbf::launch_fill_zero(d_hits, 1, st);
    if (e == hipSuccess) {
        sbf::ProbeArgs a;
        a.filter = h->d_filter;
        a.shard_mask = (uint32_t)(h->num_shards - 1);
        a.n = n;
        a.seed = seed;
        a.hits = reinterpret_cast<unsigned long long*>(d_hits);
        a.stream = st;
        e = h->ks.probe(a, h->P);
    }
    if (e != hipSuccess)
        return fail_hip(e, "probe launch");
    ok();
    return SBF_OK;
}

int sbf_fpr_probe(sbf_t* h, uint64_t n, uint64_t seed, uint64_t* hits)
{
    if (!h || !hits)
        return fail(SBF_EINVAL, "NULL argument");
    int rc = sbf_fpr_probe_device(h, n, seed, reinterpret_cast<uint64_t*>(h->d_hits), nullptr);
    if (rc)
        return rc;
    hipError_t e = hipMemcpy(hits, h->d_hits, sizeof(uint64_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail_hip(e, "probe result");
    ok();
    return SBF_OK;
}

const char* sbf_strerror(int code)
{
    switch (code) {
    case SBF_OK: return "ok";
    case SBF_EINVAL: return "invalid argument";
    case SBF_EUNSUPPORTED: return "not available for this filter";
    case SBF_ENOMEM: return "out of memory";
    case SBF_EDEVICE: return "device error";
    case SBF_EIO: return "file error";
    default: return "unknown error";
    }
}

const char* sbf_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
