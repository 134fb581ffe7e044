// sbf_host.hpp -- host-side pieces of the library: the FASTA/FASTQ reader
// and the chunked, pinned host-to-device pipeline.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

namespace sbf {

// Streaming FASTA/FASTQ reader (sbf_fastx.cpp).
struct FastxReader;
FastxReader* fastx_open(const char* path, std::string* err);
void fastx_close(FastxReader* r);
// 0 on success, -1 on a read error, -2 on malformed input (text in fastx_error).
int fastx_read(FastxReader* r, char* buf, uint64_t cap, uint64_t* len, uint64_t* ends, uint64_t ends_cap,
               uint64_t* n_ends);
uint64_t fastx_records(const FastxReader* r);
uint64_t fastx_stream_length(const FastxReader* r);  // bytes of the normalized stream so far
const std::string& fastx_error(const FastxReader* r);

// Parallel BGZF decoder (sbf_bgzf.cpp): the decompressed bytes of a BGZF file
// in order, in spans that stay valid until the next call.
struct BgzfReader;
bool bgzf_detect(const unsigned char* head, size_t n);  // the first member's header is BGZF
BgzfReader* bgzf_open(const char* path, std::string* err);
void bgzf_close(BgzfReader* r);
// 0 with *n == 0 at the end of the file; -1 on a read error or a bad member.
int bgzf_next(BgzfReader* r, const char** p, size_t* n, std::string* err);

}  // namespace sbf
