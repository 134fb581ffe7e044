// sbf_bgzf.cpp -- parallel reader of BGZF files (host code, zlib).
//
// BGZF, the blocked gzip format of the SAM/BAM format specification (§4.1
// "The BGZF compression format"), is a gzip file whose every member is an
// independent deflate stream of at most 64 KiB of data, with an extra
// subfield 'BC' in its header that holds the member's total size minus one.
// Genome references are commonly distributed compressed this way (bgzip).
// Since member boundaries can be read from the headers without inflating and
// each trailer gives the member's uncompressed size (ISIZE), members can be
// inflated by several threads at once.  A reader thread cuts the file into
// chunks of whole members (about 1 MiB compressed) in a ring of slots; a pool
// of workers inflates one chunk each; the FASTA/FASTQ parser takes the chunks
// in file order as each one completes, and its slot goes back to the reader.
//
// Every member is checked: the header fields that make it BGZF, a
// consistent block size, an inflate that ends exactly at the trailer with
// ISIZE bytes, and the CRC-32 of the output.  A member that fails any check,
// or a member cut by the end of the file, ends the stream with an error after
// the data before it.  A later gzip member that is not BGZF (another gzip
// file appended) hands the rest of the file to zlib's gzread, which the
// reader thread runs itself; bytes after the last member that do not start
// a gzip header are ignored, as zlib ignores them.
#include <zlib.h>

#include <fcntl.h>
#include <unistd.h>

#include <condition_variable>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <system_error>
#include <thread>
#include <vector>

#include "sbf_host.hpp"

namespace sbf {

namespace {

constexpr size_t kHeader = 18;           // fixed header with XLEN = 6 ('BC' subfield only)
constexpr size_t kMinMember = 12 + 6 + 8;  // header with the 'BC' subfield, trailer
constexpr uint32_t kMaxIsize = 1u << 16;  // a member holds at most 64 KiB

inline uint32_t le16(const unsigned char* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
inline uint32_t le32(const unsigned char* p) { return le16(p) | (le16(p + 2) << 16); }

// Total size of the BGZF member whose header starts at p (n bytes available,
// at least 12): 0 if the header is not BGZF, else BSIZE + 1.  *xlen gets the
// length of the extra field.
size_t member_size(const unsigned char* p, size_t n, uint32_t* xlen)
{
    if (p[0] != 0x1f || p[1] != 0x8b || p[2] != 8 || p[3] != 4)  // gzip, deflate, FLG = FEXTRA only
        return 0;
    const uint32_t xl = le16(p + 10);
    if (n < 12 + (size_t)xl)
        return 0;
    for (uint32_t o = 0; o + 4 <= xl;) {  // subfields: SI1 SI2 SLEN data
        const unsigned char* f = p + 12 + o;
        const uint32_t slen = le16(f + 2);
        if (f[0] == 'B' && f[1] == 'C' && slen == 2 && o + 6 <= xl) {
            *xlen = xl;
            return (size_t)le16(f + 4) + 1;
        }
        o += 4 + slen;
    }
    return 0;
}

struct Member {
    size_t in_off, in_len;  // deflate data within the chunk's compressed bytes
    size_t out_off;         // place of its output within the chunk's output
    uint32_t isize, crc;
};

constexpr size_t kChunk = 1u << 20;      // compressed bytes per chunk (whole members)
constexpr unsigned kTailChunk = 4u << 20;  // output bytes per chunk past the BGZF members

}  // namespace

bool bgzf_detect(const unsigned char* head, size_t n)
{
    uint32_t xl = 0;
    return n >= kHeader && member_size(head, n, &xl) >= kMinMember;
}

struct BgzfReader {
    enum class St { free, queued, done, failed };
    struct Slot {
        std::vector<unsigned char> in;
        std::vector<char> out;
        std::vector<Member> mem;
        size_t out_len = 0;
        St st = St::free;
        bool last = false;  // no chunk follows
        std::string err;
    };

    FILE* fp = nullptr;
    uint64_t foff = 0;       // file offset of the next byte fp returns
    int64_t tail_at = -1;    // offset of the first member that is not BGZF, once met
    std::vector<Slot> ring;
    std::vector<size_t> queue;  // slots waiting for a worker, oldest first
    size_t qhead = 0;

    std::mutex mu;
    std::condition_variable cv_reader, cv_work, cv_consumer;
    bool stop = false;
    uint64_t wpos = 0, rpos = 0;  // chunks cut by the reader / taken by the consumer
    bool holding = false;         // the consumer still reads chunk rpos
    bool ended = false;           // the consumer has taken the last chunk
    std::thread reader;
    std::vector<std::thread> workers;

    ~BgzfReader()
    {
        {
            std::lock_guard<std::mutex> g(mu);
            stop = true;
        }
        cv_reader.notify_all();
        cv_work.notify_all();
        cv_consumer.notify_all();
        if (reader.joinable())
            reader.join();
        for (auto& w : workers)
            if (w.joinable())
                w.join();
        if (fp)
            std::fclose(fp);
    }

    // Cut the next chunk into s: whole members until about kChunk bytes, the
    // end of the file (eof) or a member that is not BGZF (tail_at set).
    // Returns false with s.err set on a bad or cut member.
    bool cut(Slot& s, bool& eof)
    {
        s.in.clear();
        s.in.reserve(kChunk + kMaxIsize + 64);
        s.mem.clear();
        s.out_len = 0;
        s.err.clear();
        unsigned char hdr[12];
        while (s.in.size() < kChunk) {
            const uint64_t mstart = foff;
            const size_t got = std::fread(hdr, 1, sizeof hdr, fp);
            foff += got;
            if (std::ferror(fp)) {
                s.err = "read error";
                return false;
            }
            if (got == 0 || hdr[0] != 0x1f || (got > 1 && hdr[1] != 0x8b)) {
                eof = true;  // the end, or trailing bytes that are not gzip
                return true;
            }
            if (got < sizeof hdr) {
                s.err = "BGZF: truncated member at the end of the file";
                return false;
            }
            if (hdr[2] != 8 || hdr[3] != 4) {
                tail_at = (int64_t)mstart;  // a gzip member without an extra field
                return true;
            }
            const size_t o = s.in.size();
            const uint32_t xl = le16(hdr + 10);
            s.in.resize(o + 12 + xl);
            std::memcpy(s.in.data() + o, hdr, 12);
            const size_t gx = std::fread(s.in.data() + o + 12, 1, xl, fp);
            foff += gx;
            if (gx != xl) {
                s.err = "BGZF: truncated member at the end of the file";
                return false;
            }
            uint32_t xl2 = 0;
            const size_t sz = member_size(s.in.data() + o, 12 + xl, &xl2);
            if (sz == 0) {
                s.in.resize(o);
                tail_at = (int64_t)mstart;  // a gzip member without the 'BC' field
                return true;
            }
            if (sz < 12 + (size_t)xl + 8) {
                s.err = "BGZF: block size smaller than its header and trailer";
                return false;
            }
            s.in.resize(o + sz);
            const size_t gd = std::fread(s.in.data() + o + 12 + xl, 1, sz - 12 - xl, fp);
            foff += gd;
            if (gd != sz - 12 - xl) {
                s.err = "BGZF: truncated member at the end of the file";
                return false;
            }
            Member m;
            m.in_off = o + 12 + xl;
            m.in_len = sz - 12 - xl - 8;
            m.crc = le32(s.in.data() + o + sz - 8);
            m.isize = le32(s.in.data() + o + sz - 4);
            if (m.isize > kMaxIsize) {
                s.err = "BGZF: member larger than 64 KiB";
                return false;
            }
            m.out_off = s.out_len;
            s.out_len += m.isize;
            s.mem.push_back(m);
        }
        return true;
    }

    // Inflate and check every member of s.  Returns false with s.err set.
    static bool inflate_chunk(Slot& s, z_stream& z)
    {
        if (s.out.size() < s.out_len)
            s.out.resize(s.out_len);
        for (const Member& m : s.mem) {
            inflateReset(&z);
            z.next_in = s.in.data() + m.in_off;
            z.avail_in = (uInt)m.in_len;
            unsigned char spare;  // an empty member still gets a valid output pointer
            z.next_out = m.isize ? reinterpret_cast<unsigned char*>(s.out.data() + m.out_off) : &spare;
            z.avail_out = m.isize ? (uInt)m.isize : 1u;
            const int rc = inflate(&z, Z_FINISH);
            if (rc != Z_STREAM_END || z.avail_in != 0 || z.total_out != m.isize) {
                s.err = "BGZF: corrupt deflate data or wrong ISIZE";
                return false;
            }
            const uLong c =
                crc32(crc32(0L, Z_NULL, 0), reinterpret_cast<const Bytef*>(s.out.data() + m.out_off), (uInt)m.isize);
            if ((uint32_t)c != m.crc) {
                s.err = "BGZF: CRC-32 mismatch";
                return false;
            }
        }
        return true;
    }

    void read_loop()
    {
        for (bool eof = false; !eof;) {
            Slot* s;
            {
                std::unique_lock<std::mutex> g(mu);
                cv_reader.wait(g, [&] { return stop || wpos - rpos < ring.size(); });
                if (stop)
                    return;
                s = &ring[wpos % ring.size()];
            }
            bool ok;
            try {
                ok = cut(*s, eof);
            } catch (const std::bad_alloc&) {
                s->err = "host allocation failed";
                ok = false;
            }
            {
                std::lock_guard<std::mutex> g(mu);
                s->last = eof || !ok;
                if (!ok) {
                    s->st = St::failed;
                } else if (s->mem.empty()) {
                    s->st = St::done;  // nothing to inflate (the end of the file)
                } else {
                    s->st = St::queued;
                    queue.push_back(wpos % ring.size());
                }
                ++wpos;
            }
            cv_work.notify_one();
            cv_consumer.notify_all();
            if (!ok)
                return;
            if (tail_at >= 0) {
                tail_loop();
                return;
            }
        }
    }

    // The file from tail_at on, through zlib's gzread (sequential), in
    // chunks of up to kTailChunk bytes; an empty last chunk marks the end.
    void tail_loop()
    {
        gzFile gz = nullptr;
        const int fd = ::dup(::fileno(fp));
        if (fd >= 0 && ::lseek(fd, (off_t)tail_at, SEEK_SET) == (off_t)tail_at)
            gz = ::gzdopen(fd, "rb");
        if (!gz && fd >= 0)
            ::close(fd);
        for (bool end = false; !end;) {
            Slot* s;
            {
                std::unique_lock<std::mutex> g(mu);
                cv_reader.wait(g, [&] { return stop || wpos - rpos < ring.size(); });
                if (stop)
                    break;
                s = &ring[wpos % ring.size()];
            }
            s->mem.clear();
            s->err.clear();
            int n = -1;
            if (!gz) {
                s->err = "cannot reopen the file for its gzip members";
            } else {
                try {
                    if (s->out.size() < kTailChunk)
                        s->out.resize(kTailChunk);
                    n = ::gzread(gz, s->out.data(), kTailChunk);
                    int zerr = Z_OK;
                    const char* msg = ::gzerror(gz, &zerr);
                    if (n < 0) {
                        s->err = std::string("read error: ") + (msg ? msg : "?");
                    } else if (n == 0 && zerr == Z_BUF_ERROR) {
                        // the end of the input inside a gzip member
                        s->err = "truncated gzip data (the file ends inside a member)";
                        n = -1;
                    }
                } catch (const std::bad_alloc&) {
                    s->err = "host allocation failed";
                }
            }
            end = n <= 0;
            {
                std::lock_guard<std::mutex> g(mu);
                s->out_len = n > 0 ? (size_t)n : 0;
                s->st = n < 0 ? St::failed : St::done;
                s->last = end;
                ++wpos;
            }
            cv_consumer.notify_all();
        }
        if (gz)
            ::gzclose(gz);
    }

    void work_loop()
    {
        z_stream z;
        std::memset(&z, 0, sizeof z);
        const bool zok = inflateInit2(&z, -15) == Z_OK;
        for (;;) {
            Slot* s;
            {
                std::unique_lock<std::mutex> g(mu);
                cv_work.wait(g, [&] { return stop || qhead < queue.size(); });
                if (stop)
                    break;
                s = &ring[queue[qhead++]];
                if (qhead == queue.size()) {
                    queue.clear();
                    qhead = 0;
                }
            }
            bool ok = false;
            if (!zok) {
                s->err = "BGZF: inflate initialization failed";
            } else {
                try {
                    ok = inflate_chunk(*s, z);
                } catch (const std::bad_alloc&) {
                    s->err = "host allocation failed";
                }
            }
            {
                std::lock_guard<std::mutex> g(mu);
                s->st = ok ? St::done : St::failed;
            }
            cv_consumer.notify_all();
        }
        if (zok)
            inflateEnd(&z);
    }

    // Next decoded span, valid until the next call; *n == 0 at the end.  -1
    // on error (text in *err).
    int next(const char** p, size_t* n, std::string* err)
    {
        std::unique_lock<std::mutex> g(mu);
        for (;;) {
            if (holding) {  // hand the slot read last back to the reader
                Slot& s = ring[rpos % ring.size()];
                ended = s.last;
                s.st = St::free;
                holding = false;
                ++rpos;
                cv_reader.notify_one();
            }
            if (ended) {
                *p = nullptr;
                *n = 0;
                return 0;
            }
            cv_consumer.wait(g, [&] {
                const St st = ring[rpos % ring.size()].st;
                return rpos < wpos && (st == St::done || st == St::failed);
            });
            Slot& s = ring[rpos % ring.size()];
            if (s.st == St::failed) {
                *err = s.err;
                return -1;
            }
            holding = true;
            if (s.out_len == 0)
                continue;  // only empty members: take the next chunk
            *p = s.out.data();
            *n = s.out_len;
            return 0;
        }
    }
};

BgzfReader* bgzf_open(const char* path, std::string* err)
{
    BgzfReader* r = new (std::nothrow) BgzfReader();
    if (!r) {
        *err = "host allocation failed";
        return nullptr;
    }
    r->fp = std::fopen(path, "rb");
    if (!r->fp) {
        *err = std::string("cannot open ") + path;
        delete r;
        return nullptr;
    }
    // one core is the parser's; at most 16 threads in all
    const unsigned hw = std::thread::hardware_concurrency();
    const int nw = hw <= 2 ? 1 : (hw > 16 ? 15 : (int)hw - 1);
    try {
        r->ring.resize((size_t)(2 * nw + 2));
        r->reader = std::thread(&BgzfReader::read_loop, r);
        for (int i = 0; i < nw; ++i)
            r->workers.emplace_back(&BgzfReader::work_loop, r);
    } catch (...) {
        *err = "cannot start the decoding threads";
        delete r;
        return nullptr;
    }
    return r;
}

void bgzf_close(BgzfReader* r) { delete r; }

int bgzf_next(BgzfReader* r, const char** p, size_t* n, std::string* err) { return r->next(p, n, err); }

}  // namespace sbf
