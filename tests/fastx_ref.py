"""Reference FASTA/FASTQ normalization for the tests, written from the rules
in include/sbf.h (and [cuSBF] §IV-F: records joined by one 'N'), line by line
in Python.  Independent of the library's streaming reader."""


def _lines(text: bytes):
    for raw in text.split(b"\n"):
        line = raw.lstrip(b"\r")
        if line:
            yield line


def _seq(line: bytes) -> bytes:
    return bytes(c for c in line if c > 0x20)


def normalize(text: bytes):
    """(normalized stream, record end offsets) of a FASTA/FASTQ file's bytes."""
    lines = list(_lines(text))
    if not lines:
        return b"", []
    recs = []
    if lines[0][:1] == b">":
        cur = None
        for line in lines:
            if line[:1] == b">":
                if cur is not None:
                    recs.append(b"".join(cur))
                cur = []
            elif line[:1] == b";":
                continue
            else:
                cur.append(_seq(line))
        if cur is not None:
            recs.append(b"".join(cur))
    elif lines[0][:1] == b"@":
        i = 0
        while i < len(lines):
            assert lines[i][:1] == b"@", "malformed FASTQ"
            i += 1
            seq = []
            while i < len(lines) and lines[i][:1] != b"+":
                seq.append(_seq(lines[i]))
                i += 1
            assert i < len(lines), "truncated FASTQ"
            i += 1  # '+' line
            s = b"".join(seq)
            q = 0
            while q < len(s):
                assert i < len(lines), "truncated FASTQ"
                q += len(_seq(lines[i]))
                i += 1
            recs.append(s)
    else:
        raise ValueError("not FASTA or FASTQ")
    ends, pos = [], 0
    for r in recs:
        pos += len(r)
        ends.append(pos)
        pos += 1
    return b"N".join(recs), ends
