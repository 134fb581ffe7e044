// sbf_fastx.cpp -- streaming FASTA/FASTQ reader (host code, zlib).
//
// [cuSBF] §IV-A lists streamed FASTA/FASTQ input with transparent gzip
// decompression among the input forms, and §IV-F fixes how records become one
// sequence: consecutive records are joined by an invalid separator ('N' for
// DNA), so every k-mer that spans a record boundary is invalid and no kernel
// tracks boundaries.  The reader produces that "normalized stream": each
// record's sequence with line breaks and other whitespace removed, records
// joined by one 'N', plus the stream offset at which each record ends.
//
// Formats (detected from the first byte that is not a line break):
//   FASTA  '>' header line, then sequence lines up to the next '>'; lines
//          starting with ';' are comments.
//   FASTQ  '@' header, sequence lines up to a line starting with '+', then
//          quality lines until as many quality bytes as bases were read (so
//          a quality line may itself start with '@').
// gzip (also multi-member) and plain files are read through zlib's gzread,
// which passes plain data through unchanged; BGZF files (gzip members of at
// most 64 KiB that state their own size) are inflated by several threads at
// once (sbf_bgzf.cpp).
#include <zlib.h>

#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/sbf.h"
#include "sbf_host.hpp"

namespace sbf {

namespace {

enum class Fmt { unknown, fasta, fastq };
enum class State { line_start, skip_line, seq, qual };

}  // namespace

struct FastxReader {
    gzFile f = nullptr;
    BgzfReader* bg = nullptr;  // set for BGZF input, which bypasses gzread
    std::vector<char> in;
    const char* inp = nullptr;  // current input span: in.data() or a BGZF batch
    size_t pos = 0, lim = 0;
    bool eof = false, finished = false;
    Fmt fmt = Fmt::unknown;
    State state = State::line_start;
    bool rec_open = false;    // a record has started and not yet ended
    bool pending_sep = false;  // the 'N' before the next record's first base is owed
    bool fq_in_qual = false;   // FASTQ: between the '+' line and the record's end
    bool fq_header_next = true;  // FASTQ: the next line must be an '@' header
    uint64_t nrec = 0;         // records started
    uint64_t total = 0;        // bytes of the normalized stream emitted
    uint64_t fq_seq = 0, fq_qual = 0;  // FASTQ bases / quality bytes of the current record
    std::string error;

    int refill()
    {
        if (eof)
            return 0;
        if (bg) {
            const char* p = nullptr;
            size_t n = 0;
            if (bgzf_next(bg, &p, &n, &error))
                return -1;
            inp = p;
            pos = 0;
            lim = n;
            if (n == 0)
                eof = true;
            return 0;
        }
        inp = in.data();
        const int got = gzread(f, in.data(), (unsigned)in.size());
        if (got < 0) {
            int zerr = 0;
            const char* msg = gzerror(f, &zerr);
            error = std::string("read error: ") + (msg ? msg : "?");
            return -1;
        }
        pos = 0;
        lim = (size_t)got;
        if (got == 0) {
            // gzread reports a file that ends inside a gzip member as the end
            // of the input, with Z_BUF_ERROR left in gzerror
            int zerr = Z_OK;
            gzerror(f, &zerr);
            if (zerr == Z_BUF_ERROR) {
                error = "truncated gzip data (the file ends inside a member)";
                return -1;
            }
            eof = true;
        }
        return 0;
    }

    // Start a record: the separator before it (none before the first).
    void start_record()
    {
        if (nrec > 0)
            pending_sep = true;
        ++nrec;
        rec_open = true;
    }
};

namespace {

// Copy bytes dropping whitespace and control bytes (<= 0x20); returns bytes written.
size_t copy_sequence(char* dst, const char* src, size_t n)
{
    std::memcpy(dst, src, n);
    unsigned char any = 0;
    for (size_t i = 0; i < n; ++i)
        any |= (unsigned char)((unsigned char)dst[i] <= 0x20);
    if (!any)
        return n;
    size_t o = 0;
    for (size_t i = 0; i < n; ++i)
        if ((unsigned char)src[i] > 0x20)
            dst[o++] = src[i];
    return o;
}

size_t count_nonspace(const char* p, size_t n)
{
    size_t c = 0;
    for (size_t i = 0; i < n; ++i)
        c += (unsigned char)p[i] > 0x20;
    return c;
}

}  // namespace

// Fill buf with up to cap bytes of the normalized stream.  Record ends go to
// ends (if not NULL); the call returns early rather than lose one when ends is
// full.  *len == 0 and *n_ends == 0 together mean the stream is finished.
int fastx_read(FastxReader* r, char* buf, uint64_t cap, uint64_t* len, uint64_t* ends, uint64_t ends_cap,
               uint64_t* n_ends)
{
    uint64_t o = 0, n = 0;
    auto end_record = [&]() -> bool {  // false: no room to report it
        if (ends && n == ends_cap)
            return false;
        if (ends)
            ends[n] = r->total;
        ++n;
        r->rec_open = false;
        return true;
    };
    while (!r->finished) {
        if (r->pending_sep) {
            if (o == cap)
                break;
            buf[o++] = 'N';
            ++r->total;
            r->pending_sep = false;
        }
        if (r->pos == r->lim) {
            if (r->refill())
                return -1;
            if (r->pos == r->lim) {  // end of input
                if (r->fmt == Fmt::fastq && r->rec_open && !(r->fq_in_qual && r->fq_qual >= r->fq_seq)) {
                    r->error = "truncated FASTQ record (quality shorter than sequence)";
                    return -2;
                }
                if (r->rec_open && !end_record())
                    break;
                r->finished = true;
                break;
            }
        }
        const char* p = r->inp + r->pos;
        const size_t avail = r->lim - r->pos;
        switch (r->state) {
        case State::line_start: {
            const char c = p[0];
            if (c == '\n' || c == '\r') {
                ++r->pos;
                continue;
            }
            if (r->fmt == Fmt::unknown) {
                if (c == '>')
                    r->fmt = Fmt::fasta;
                else if (c == '@')
                    r->fmt = Fmt::fastq;
                else {
                    r->error = "not FASTA or FASTQ (first byte is neither '>' nor '@')";
                    return -2;
                }
            }
            if (r->fmt == Fmt::fasta) {
                if (c == '>') {
                    if (r->rec_open && !end_record())
                        goto out;
                    r->start_record();
                    r->state = State::skip_line;
                    ++r->pos;
                } else if (c == ';') {
                    r->state = State::skip_line;
                    ++r->pos;
                } else {
                    if (!r->rec_open)
                        r->start_record();
                    r->state = State::seq;
                }
            } else {
                if (r->fq_header_next) {
                    if (c != '@') {
                        r->error = "malformed FASTQ: expected a '@' header line";
                        return -2;
                    }
                    if (r->rec_open && !end_record())
                        goto out;
                    r->start_record();
                    r->fq_header_next = false;
                    r->fq_in_qual = false;
                    r->fq_seq = r->fq_qual = 0;
                    r->state = State::skip_line;
                    ++r->pos;
                } else if (!r->fq_in_qual) {
                    if (c == '+') {
                        r->fq_in_qual = true;
                        r->state = State::skip_line;
                        ++r->pos;
                        if (r->fq_seq == 0)
                            r->fq_header_next = true;  // empty record: no quality lines follow
                    } else {
                        r->state = State::seq;
                    }
                } else {
                    r->state = State::qual;
                }
            }
            break;
        }
        case State::skip_line: {
            const char* nl = static_cast<const char*>(std::memchr(p, '\n', avail));
            if (nl) {
                r->pos += (size_t)(nl - p) + 1;
                r->state = State::line_start;
            } else {
                r->pos = r->lim;
            }
            break;
        }
        case State::seq: {
            const char* nl = static_cast<const char*>(std::memchr(p, '\n', avail));
            const size_t seg = nl ? (size_t)(nl - p) : avail;
            const uint64_t room = cap - o;
            const size_t take = seg < room ? seg : (size_t)room;
            const size_t w = copy_sequence(buf + o, p, take);
            o += w;
            r->total += w;
            r->fq_seq += w;
            r->pos += take;
            if (take < seg)
                goto out;  // output full
            if (nl) {
                ++r->pos;
                r->state = State::line_start;
            }
            break;
        }
        case State::qual: {
            const char* nl = static_cast<const char*>(std::memchr(p, '\n', avail));
            const size_t seg = nl ? (size_t)(nl - p) : avail;
            r->fq_qual += count_nonspace(p, seg);
            r->pos += seg;
            if (nl) {
                ++r->pos;
                r->state = State::line_start;
                if (r->fq_qual >= r->fq_seq)
                    r->fq_header_next = true;
            }
            break;
        }
        }
        if (o == cap && !r->pending_sep && r->state == State::seq)
            break;
    }
out:
    *len = o;
    *n_ends = n;
    return 0;
}

FastxReader* fastx_open(const char* path, std::string* err)
{
    unsigned char head[18];
    size_t nhead = 0;
    if (FILE* fp = std::fopen(path, "rb")) {
        nhead = std::fread(head, 1, sizeof head, fp);
        std::fclose(fp);
    }
    if (bgzf_detect(head, nhead)) {
        BgzfReader* bg = bgzf_open(path, err);
        if (!bg)
            return nullptr;
        FastxReader* r = new (std::nothrow) FastxReader();
        if (!r) {
            bgzf_close(bg);
            *err = "host allocation failed";
            return nullptr;
        }
        r->bg = bg;
        return r;
    }
    gzFile f = gzopen(path, "rb");
    if (!f) {
        *err = std::string("cannot open ") + path;
        return nullptr;
    }
    gzbuffer(f, 1u << 20);
    FastxReader* r = new (std::nothrow) FastxReader();
    if (!r) {
        gzclose(f);
        *err = "host allocation failed";
        return nullptr;
    }
    r->f = f;
    try {
        r->in.resize(1u << 22);
    } catch (...) {
        gzclose(f);
        delete r;
        *err = "host allocation failed";
        return nullptr;
    }
    return r;
}

void fastx_close(FastxReader* r)
{
    if (!r)
        return;
    if (r->f)
        gzclose(r->f);
    if (r->bg)
        bgzf_close(r->bg);
    delete r;
}

uint64_t fastx_records(const FastxReader* r) { return r->nrec; }
uint64_t fastx_stream_length(const FastxReader* r) { return r->total; }
const std::string& fastx_error(const FastxReader* r) { return r->error; }

}  // namespace sbf
