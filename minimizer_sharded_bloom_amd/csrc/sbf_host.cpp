// sbf_host.cpp -- host-resident input: the chunked, double-buffered
// host-to-device pipeline and the FASTA/FASTQ entry points.
//
// [cuSBF] §IV-G (host FASTX staging): multi-chunk workloads overlap host
// normalization, pinned staging and host-to-device copies with GPU work on
// alternating streams.  Here a chunk is up to `chunk` k-mer starts plus the
// k-1 bases that the last of them reaches; consecutive chunks overlap by k-1
// bases, so every k-mer start belongs to exactly one chunk.  Slot b (b = chunk
// index mod kHostSlots) owns a pinned buffer, device buffers and a stream.
// While the copies, pack, insert or query and answer copy of the other slots
// run, the host fills the next slot (a copy from the caller's memory, or the
// FASTX reader writing the normalized stream straight into pinned memory).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <mutex>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "../../include/sbf.h"
#include "sbf_handle.hpp"
#include "sbf_host.hpp"

namespace sbf {

namespace {

uint64_t words_for(uint64_t nk) { return (nk + 63) / 64; }

double now_s()
{
    return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// Persistent copy threads: a large pageable -> pinned copy is split into
// parts taken by the caller and the workers (at most 16 threads in all).
class CopyPool {
public:
    static CopyPool& get()
    {
        static CopyPool pool;
        return pool;
    }
    void copy(char* dst, const char* src, uint64_t n)
    {
        const uint64_t kPart = 4ull << 20;
        if (workers_.empty() || n < 2 * kPart) {
            std::memcpy(dst, src, n);
            return;
        }
        std::unique_lock<std::mutex> lk(mu_);
        dst_ = dst;
        src_ = src;
        n_ = n;
        part_ = std::max<uint64_t>(kPart, (n + 4 * nthreads() - 1) / (4 * nthreads()));
        nparts_ = (n + part_ - 1) / part_;
        next_.store(0);
        left_ = nparts_;
        ++gen_;
        lk.unlock();
        cv_.notify_all();
        work();
        lk.lock();
        // every part copied and no worker still inside work(), so the next
        // job may rewrite the job fields
        done_.wait(lk, [&] { return left_ == 0 && active_ == 0; });
    }

private:
    CopyPool()
    {
        unsigned hw = std::thread::hardware_concurrency();
        const unsigned t = std::min(16u, hw ? hw : 1u);
        for (unsigned i = 1; i < t; ++i)
            workers_.emplace_back([this] { loop(); });
    }
    ~CopyPool()
    {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : workers_)
            t.join();
    }
    unsigned nthreads() const { return (unsigned)workers_.size() + 1; }
    void work()
    {
        uint64_t done = 0;
        for (;;) {
            const uint64_t i = next_.fetch_add(1);
            if (i >= nparts_)
                break;
            const uint64_t a = i * part_, b = std::min(n_, a + part_);
            std::memcpy(dst_ + a, src_ + a, b - a);
            ++done;
        }
        if (done) {
            std::lock_guard<std::mutex> lk(mu_);
            left_ -= done;
            if (left_ == 0)
                done_.notify_all();
        }
    }
    void loop()
    {
        uint64_t seen = 0;
        for (;;) {
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
                if (stop_)
                    return;
                seen = gen_;
                ++active_;
            }
            work();
            std::lock_guard<std::mutex> lk(mu_);
            if (--active_ == 0)
                done_.notify_all();
        }
    }
    std::vector<std::thread> workers_;
    std::mutex mu_;
    std::condition_variable cv_, done_;
    char* dst_ = nullptr;
    const char* src_ = nullptr;
    uint64_t n_ = 0, part_ = 0, nparts_ = 0, left_ = 0, gen_ = 0;
    unsigned active_ = 0;  // workers inside work()
    std::atomic<uint64_t> next_{0};
    bool stop_ = false;
};

int ensure_staging(sbf_t* h)
{
    HostStaging& hs = h->host;
    if (hs.built_for == hs.chunk && hs.s[0])
        return SBF_OK;
    free_host_staging(hs);
    // + k-1 <= 31 symbols of overlap, padded; a triplet symbol is 3 bytes
    const uint64_t in_bytes = (hs.chunk + 64) * symbol_bytes(h);
    const uint64_t out_words = hs.chunk / 64 + 1;
    hipError_t e = hipSuccess;
    for (int b = 0; b < kHostSlots && e == hipSuccess; ++b) {
        e = hipStreamCreateWithFlags(&hs.s[b], hipStreamNonBlocking);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&hs.done[b], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipHostMalloc(reinterpret_cast<void**>(&hs.h_in[b]), in_bytes, hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipHostMalloc(reinterpret_cast<void**>(&hs.h_out[b]), 8 * out_words, hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void**>(&hs.d_in[b]), in_bytes);
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void**>(&hs.d_codes[b]), 4 * ((in_bytes + 15) / 16));
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void**>(&hs.d_valid[b]), 4 * ((in_bytes + 31) / 32));
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void**>(&hs.d_out[b]), 8 * out_words);
    }
    if (e != hipSuccess) {
        free_host_staging(hs);
        return fail_hip(e, "host staging buffers");
    }
    hs.built_for = hs.chunk;
    return SBF_OK;
}

// Producer of the sequence bytes, in order.
struct Source {
    virtual ~Source() = default;
    // Write up to cap bytes to dst; *got = 0 at the end.  Returns SBF_OK or
    // an SBF_E* code (with the error text set).
    virtual int next(char* dst, uint64_t cap, uint64_t* got) = 0;
};

// Receiver of one finished query chunk: answers for k-mer starts
// [first, first + nk) of the stream, LSB-first words.
struct Sink {
    virtual ~Sink() = default;
    virtual void chunk(uint64_t first, uint64_t nk, const uint64_t* words) = 0;
};

struct Slot {
    bool busy = false;
    uint64_t first = 0, nk = 0;
};

// Run the pipeline over src: insert (sink == NULL) or query into sink.
int run_pipeline(sbf_t* h, Source& src, Sink* sink, hipStream_t user, uint64_t* chunks_out, double* src_seconds)
{
    int rc = ensure_staging(h);
    if (rc)
        return rc;
    HostStaging& hs = h->host;
    const uint64_t k = h->P.k;
    const uint64_t sb = symbol_bytes(h);  // bytes per symbol
    const uint64_t want = (hs.chunk + k - 1) * sb;
    // order after the caller's earlier work on `user`
    hipEvent_t start;
    hipError_t e = hipEventCreateWithFlags(&start, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventRecord(start, user);
    for (int b = 0; b < kHostSlots && e == hipSuccess; ++b)
        e = hipStreamWaitEvent(hs.s[b], start, 0);
    if (e != hipSuccess) {
        (void)hipEventDestroy(start);
        return fail_hip(e, "pipeline start");
    }
    Slot slot[kHostSlots];
    uint64_t first = 0;    // stream offset of the next chunk's first byte
    uint64_t carry = 0;    // bytes at the front of the next chunk copied from the previous one
    const char* carry_src = nullptr;
    uint64_t nchunks = 0;
    double t_src = 0;
    bool ended = false;
    rc = SBF_OK;
    auto drain = [&](int b) -> hipError_t {
        if (!slot[b].busy)
            return hipSuccess;
        hipError_t r = hipEventSynchronize(hs.done[b]);
        if (r == hipSuccess && sink)
            sink->chunk(slot[b].first, slot[b].nk, hs.h_out[b]);
        slot[b].busy = false;
        return r;
    };
    for (uint64_t i = 0; !ended; ++i) {
        const int b = (int)(i % kHostSlots);
        e = drain(b);
        if (e != hipSuccess)
            break;
        char* dst = hs.h_in[b];
        uint64_t have = 0;
        if (carry) {
            std::memmove(dst, carry_src, carry);
            have = carry;
        }
        const double t0 = now_s();
        while (have < want) {
            uint64_t got = 0;
            rc = src.next(dst + have, want - have, &got);
            if (rc)
                break;
            if (got == 0) {
                ended = true;
                break;
            }
            have += got;
        }
        t_src += now_s() - t0;
        if (rc)
            break;
        const uint64_t nsym = have / sb;
        if (nsym < k)
            break;  // no k-mer starts left
        const uint64_t nk = nsym - k + 1;
        const hipStream_t s = hs.s[b];
        e = hipMemcpyAsync(hs.d_in[b], dst, have, hipMemcpyHostToDevice, s);
        if (e == hipSuccess && h->P.alpha != SBF_ALPHABET_DNA) {
            const SeqArgs a = text_args(h, hs.d_in[b], have, sink ? hs.d_out[b] : nullptr, s);
            e = sink ? h->ks.query(a, h->P) : h->ks.insert(a, h->P);
        } else if (e == hipSuccess && sink && h->ks.query_text) {
            // DNA query read as ASCII by the query kernel itself
            e = h->ks.query_text(text_args(h, hs.d_in[b], have, hs.d_out[b], s), h->P);
        } else if (e == hipSuccess) {
            e = launch_pack(hs.d_in[b], have, hs.d_codes[b], hs.d_valid[b], s);
            if (e == hipSuccess) {
                const SeqArgs a = seq_args(h, hs.d_codes[b], hs.d_valid[b], have, sink ? hs.d_out[b] : nullptr, s);
                e = sink ? h->ks.query(a, h->P) : h->ks.insert(a, h->P);
            }
        }
        if (e == hipSuccess && sink)
            e = hipMemcpyAsync(hs.h_out[b], hs.d_out[b], 8 * words_for(nk), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess)
            e = hipEventRecord(hs.done[b], s);
        if (e != hipSuccess)
            break;
        slot[b].busy = true;
        slot[b].first = first;
        slot[b].nk = nk;
        ++nchunks;
        // the next chunk starts at the k-mer after this chunk's last one
        // (have = want, a whole number of symbols, unless the input ended)
        carry = (k - 1) * sb;
        carry_src = dst + nsym * sb - carry;
        first += nk;
    }
    // drain both slots (oldest first) even after an error, so no copy still
    // targets the pinned buffers
    for (uint64_t j = nchunks >= kHostSlots ? nchunks - kHostSlots : 0; j < nchunks; ++j) {
        const hipError_t e2 = drain((int)(j % kHostSlots));
        if (e == hipSuccess)
            e = e2;
    }
    (void)hipEventDestroy(start);
    if (rc)
        return rc;
    if (e != hipSuccess)
        return fail_hip(e, "host pipeline");
    if (chunks_out)
        *chunks_out = nchunks;
    if (src_seconds)
        *src_seconds = t_src;
    ok();
    return SBF_OK;
}

// Host memory -> pinned staging.
struct MemSource : Source {
    const char* p;
    uint64_t left;
    MemSource(const char* q, uint64_t n) : p(q), left(n) {}
    int next(char* dst, uint64_t cap, uint64_t* got) override
    {
        const uint64_t n = std::min(cap, left);
        CopyPool::get().copy(dst, p, n);
        p += n;
        left -= n;
        *got = n;
        return 0;
    }
};

// Answer words -> the caller's bit vector.  Chunks hold a multiple of 64 k-mer
// starts except the last, so every chunk starts on a word boundary.
struct BitsSink : Sink {
    uint64_t* out;
    explicit BitsSink(uint64_t* o) : out(o) {}
    void chunk(uint64_t first, uint64_t nk, const uint64_t* words) override
    {
        std::memcpy(out + first / 64, words, 8 * words_for(nk));
    }
};

// FASTX reader -> pinned staging; record ends kept when asked for.
struct FastxSource : Source {
    FastxReader* r;
    std::vector<uint64_t>* ends;  // may be NULL
    uint64_t tmp[4096];
    explicit FastxSource(FastxReader* rd, std::vector<uint64_t>* e) : r(rd), ends(e) {}
    int next(char* dst, uint64_t cap, uint64_t* got) override
    {
        for (;;) {
            uint64_t len = 0, n = 0;
            const int rc = fastx_read(r, dst, cap, &len, ends ? tmp : nullptr, ends ? 4096 : 0, &n);
            if (rc)
                return fail(SBF_EIO, fastx_error(r).c_str());
            if (ends)
                ends->insert(ends->end(), tmp, tmp + n);
            if (len || !n) {  // bytes, or the end of the stream
                *got = len;
                return 0;
            }
        }
    }
};

uint64_t popcount_range(const uint64_t* w, uint64_t a, uint64_t b)  // bits [a, b)
{
    uint64_t c = 0;
    while (a < b && (a & 63)) {
        c += (w[a >> 6] >> (a & 63)) & 1u;
        ++a;
    }
    for (; a + 64 <= b; a += 64)
        c += (uint64_t)__builtin_popcountll(w[a >> 6]);
    for (; a < b; ++a)
        c += (w[a >> 6] >> (a & 63)) & 1u;
    return c;
}

// Per-record counts: hits[r] = present k-mers of record r, kmers[r] = its
// k-mer starts.  Record r spans [start_r, end_r) of the normalized stream,
// start_0 = 0 and start_r = end_{r-1} + 1; its k-mers start in
// [start_r, end_r - k]; a k-mer starting later reaches the separator and
// answers 0, so counting answer bits over [start_r, end_r) is exact.
struct RecordSink : Sink {
    const std::vector<uint64_t>& ends;
    uint64_t k;
    uint64_t* hits;
    uint64_t* kmers;
    uint64_t cap;
    uint64_t cur = 0;       // first record not yet complete
    uint64_t cur_hits = 0;  // its hits so far
    RecordSink(const std::vector<uint64_t>& e, uint64_t kk, uint64_t* h, uint64_t* km, uint64_t c)
        : ends(e), k(kk), hits(h), kmers(km), cap(c) {}
    uint64_t start_of(uint64_t r) const { return r == 0 ? 0 : ends[r - 1] + 1; }
    void finish(uint64_t r)
    {
        if (r < cap) {
            const uint64_t len = ends[r] - start_of(r);
            if (hits)
                hits[r] = cur_hits;
            if (kmers)
                kmers[r] = len >= k ? len - k + 1 : 0;
        }
        cur_hits = 0;
    }
    void chunk(uint64_t first, uint64_t nk, const uint64_t* words) override
    {
        const uint64_t last = first + nk;
        for (;;) {
            // every record ending before `last` is known: the reader has
            // already produced the following chunk
            const bool known = cur < ends.size();
            const uint64_t s = std::max(start_of(cur), first);
            const uint64_t e = known ? std::min(ends[cur], last) : last;
            if (s < e)
                cur_hits += popcount_range(words, s - first, e - first);
            if (known && ends[cur] <= last) {
                finish(cur);
                ++cur;
                continue;
            }
            break;
        }
    }
    void close()
    {
        while (cur < ends.size()) {  // records without k-mers after the last chunk
            finish(cur);
            ++cur;
        }
    }
};

}  // namespace

void free_host_staging(HostStaging& hs)
{
    for (int b = 0; b < kHostSlots; ++b) {
        if (hs.s[b])
            (void)hipStreamSynchronize(hs.s[b]);
        if (hs.h_in[b])
            (void)hipHostFree(hs.h_in[b]);
        if (hs.h_out[b])
            (void)hipHostFree(hs.h_out[b]);
        if (hs.d_in[b])
            (void)hipFree(hs.d_in[b]);
        if (hs.d_codes[b])
            (void)hipFree(hs.d_codes[b]);
        if (hs.d_valid[b])
            (void)hipFree(hs.d_valid[b]);
        if (hs.d_out[b])
            (void)hipFree(hs.d_out[b]);
        if (hs.done[b])
            (void)hipEventDestroy(hs.done[b]);
        if (hs.s[b])
            (void)hipStreamDestroy(hs.s[b]);
        hs.s[b] = nullptr;
        hs.done[b] = nullptr;
        hs.h_in[b] = nullptr;
        hs.h_out[b] = nullptr;
        hs.d_in[b] = nullptr;
        hs.d_codes[b] = nullptr;
        hs.d_valid[b] = nullptr;
        hs.d_out[b] = nullptr;
    }
    hs.built_for = 0;
}

int host_insert(sbf_t* h, const char* seq, uint64_t len, hipStream_t st)
{
    MemSource src(seq, len);
    return run_pipeline(h, src, nullptr, st, nullptr, nullptr);
}

int host_query(sbf_t* h, const char* seq, uint64_t len, uint64_t* out_bits, hipStream_t st)
{
    MemSource src(seq, len);
    BitsSink sink(out_bits);
    return run_pipeline(h, src, &sink, st, nullptr, nullptr);
}

}  // namespace sbf

struct sbf_fastx {
    sbf::FastxReader* r;
};

extern "C" {

int sbf_set_staging(sbf_t* h, uint64_t chunk_bases)
{
    if (!h)
        return sbf::fail(SBF_EINVAL, "handle is NULL");
    if (chunk_bases < 64 || chunk_bases > (1ull << 34))
        return sbf::fail(SBF_EINVAL, "chunk_bases must be in 64..2^34");
    int rc = sbf::set_device(h);
    if (rc)
        return rc;
    h->host.chunk = (chunk_bases + 63) & ~63ull;
    if (h->host.built_for && h->host.built_for != h->host.chunk)
        sbf::free_host_staging(h->host);
    sbf::ok();
    return SBF_OK;
}

int sbf_fastx_open(sbf_fastx_t** out, const char* path)
{
    if (!out || !path)
        return sbf::fail(SBF_EINVAL, "NULL argument");
    std::string err;
    sbf::FastxReader* r = sbf::fastx_open(path, &err);
    if (!r)
        return sbf::fail(SBF_EIO, err.c_str());
    sbf_fastx_t* f = new (std::nothrow) sbf_fastx_t{r};
    if (!f) {
        sbf::fastx_close(r);
        return sbf::fail(SBF_ENOMEM, "host allocation failed");
    }
    *out = f;
    sbf::ok();
    return SBF_OK;
}

int sbf_fastx_read(sbf_fastx_t* f, char* buf, uint64_t cap, uint64_t* len, uint64_t* ends, uint64_t ends_cap,
                   uint64_t* n_ends)
{
    if (!f || !buf || !len || !n_ends || cap == 0 || (ends && ends_cap == 0))
        return sbf::fail(SBF_EINVAL, "bad argument");
    const int rc = sbf::fastx_read(f->r, buf, cap, len, ends, ends_cap, n_ends);
    if (rc)
        return sbf::fail(SBF_EIO, sbf::fastx_error(f->r).c_str());
    sbf::ok();
    return SBF_OK;
}

uint64_t sbf_fastx_records(const sbf_fastx_t* f) { return f ? sbf::fastx_records(f->r) : 0; }

int sbf_fastx_close(sbf_fastx_t* f)
{
    if (f) {
        sbf::fastx_close(f->r);
        delete f;
    }
    sbf::ok();
    return SBF_OK;
}

int sbf_insert_fastx(sbf_t* h, const char* path, sbf_fastx_stats_t* stats)
{
    if (!h || !path)
        return sbf::fail(SBF_EINVAL, "NULL argument");
    if (h->P.alpha != SBF_ALPHABET_DNA)
        return sbf::fail(SBF_EUNSUPPORTED, "FASTA/FASTQ input is DNA only");
    int rc = sbf::set_device(h);
    if (rc)
        return rc;
    const double t0 = sbf::now_s();
    std::string err;
    sbf::FastxReader* r = sbf::fastx_open(path, &err);
    if (!r)
        return sbf::fail(SBF_EIO, err.c_str());
    sbf::FastxSource src(r, nullptr);
    uint64_t chunks = 0;
    double t_src = 0;
    rc = sbf::run_pipeline(h, src, nullptr, nullptr, &chunks, &t_src);
    if (rc == SBF_OK && stats) {
        stats->records = sbf::fastx_records(r);
        stats->bases = sbf::fastx_stream_length(r);
        stats->chunks = chunks;
        stats->parse_seconds = t_src;
        stats->total_seconds = sbf::now_s() - t0;
    }
    sbf::fastx_close(r);
    return rc;
}

int sbf_query_fastx(sbf_t* h, const char* path, uint64_t* hits, uint64_t* kmers, uint64_t cap,
                    sbf_fastx_stats_t* stats)
{
    if (!h || !path || (cap && !hits && !kmers))
        return sbf::fail(SBF_EINVAL, "bad argument");
    if (h->P.alpha != SBF_ALPHABET_DNA)
        return sbf::fail(SBF_EUNSUPPORTED, "FASTA/FASTQ input is DNA only");
    int rc = sbf::set_device(h);
    if (rc)
        return rc;
    const double t0 = sbf::now_s();
    std::string err;
    sbf::FastxReader* r = sbf::fastx_open(path, &err);
    if (!r)
        return sbf::fail(SBF_EIO, err.c_str());
    std::vector<uint64_t> ends;
    sbf::FastxSource src(r, &ends);
    sbf::RecordSink sink(ends, h->P.k, hits, kmers, cap);
    uint64_t chunks = 0;
    double t_src = 0;
    rc = sbf::run_pipeline(h, src, &sink, nullptr, &chunks, &t_src);
    if (rc == SBF_OK) {
        sink.close();
        if (stats) {
            stats->records = sbf::fastx_records(r);
            stats->bases = sbf::fastx_stream_length(r);
            stats->chunks = chunks;
            stats->parse_seconds = t_src;
            stats->total_seconds = sbf::now_s() - t0;
        }
    }
    sbf::fastx_close(r);
    return rc;
}

}  // extern "C"
