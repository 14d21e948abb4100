"""Oracle codec: the lossless BF16 weight format, written out plainly in numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Cloudflare blog post "Unweight" (unweight-tensor-compression).
  * BF16 anatomy paragraph: a BF16 value is sign (1 bit), exponent (8 bits), mantissa
    (7 bits); sign and mantissa behave like random data and are stored unchanged.
  * Exponent-distribution paragraph and figure ("distribution of exponent values in a
    typical LLM layer"): the 16 most frequent exponents cover more than 99 % of a layer's
    weights; the exponent carries about 2.6 bits of information.
  * Huffman paragraph: only the exponent byte is entropy coded, with a Huffman code
    (short codes for common values); sign and mantissa are left as they are.
  * Rare-exponent paragraph: a row of 64 weights holding an exponent outside the top-16
    palette is stored verbatim, so the hot path takes one decision per row instead of a
    per-element branch.
  * Four-pipeline paragraphs: the direct-palette format pre-transcodes the exponents to
    4-bit palette indices at model load; a transcode pipeline produces the same indices
    from the Huffman stream at run time; an exponent-only pipeline produces exponent
    bytes; the full pipeline rebuilds BF16.
  * SM-split paragraph: the Huffman decoder's lookup table needs up to 16 KB.

Readings taken where the post is silent or garbled (each is repeated where it is used):
  R1  "row of 64 weights" = 64 consecutive weights of one matrix row along K (a segment).
  R2  A verbatim segment keeps its sign+mantissa bytes in the common stream and stores its
      64 raw exponent bytes in a side stream (the matmul paragraph stages "verbatim
      exponent rows").
  R3  Palette = the min(16, #distinct) exponents with the highest whole-matrix counts,
      ties broken toward the smaller exponent; palette index order = ascending exponent.
  R4  The Huffman alphabet is the palette index; only symbols of non-verbatim segments are
      coded; frequencies are counted over exactly those symbols.
  R5  The code is an optimal length-limited prefix code with maximum length 13 (a 2**13
      entry table, the post's "up to 16 KB" LUT at 2 bytes an entry), built by
      package-merge with fixed tie rules, then made canonical.
  R6  Bits are written MSB-first into 32-bit little-endian words.
  R7  The stream is cut into chunks of at most S coded symbols (S a multiple of 64) so
      chunks can be decoded in parallel (per-chunk start bit offsets "off"); chunks restart
      at every 64-column block of every 16-row tile, so a chunk's output never leaves one
      block and a decoder places it from that block's verbatim flags alone (per-tile first
      chunk "cbase"; inside a tile, block b holds ceil(64 * coded segments of b / S)
      chunks).
  R8  Layout: weights are grouped in tiles of 16 rows; inside a tile the sign+mantissa,
      exponent and index streams are stored as 16x16 sub-tiles (row-major inside the
      sub-tile) ordered by K; segments are enumerated in (tile, 64-column block, row) order.
  R15 The encoder may take its palette from the caller instead of the matrix's own
      histogram (ascending exponents, at most 16); the post describes only the per-matrix
      top-16, so this changes that single step and nothing after it.
"""
from __future__ import annotations

import struct

import numpy as np

TILE_ROWS = 16          # rows per tile (R8)
SEG = 64                # weights per verbatim segment along K (R1)
KSUB = 16               # columns per sub-tile (R8)
LMAX = 12               # the encoder's Huffman code length limit (R5)
LMAX_FORMAT = 13        # the longest code a blob may hold: decoders take codes up to this (R5)
DEFAULT_CHUNK = 512     # coded symbols per chunk (R7)
PALETTE_SIZE = 16       # top-16 exponents (exponent-distribution paragraph)
NONE = 0xFF             # index_of[] value for an exponent outside the palette
MAGIC = b"UW1\0"
VERSION = 1
HEADER_BYTES = 256
ALIGN = 256
SECTION_NAMES = ("sm", "flags", "vprefix", "vexp", "cbase", "off", "words")


# ----------------------------------------------------------------------------------------
# BF16 field split (BF16 anatomy paragraph)
# ----------------------------------------------------------------------------------------
def split_fields(w):
    """w: uint16 BF16 bit patterns -> (exponent byte e, sign+mantissa byte sm).

    e = bits 14..7; sm = sign bit in bit 7, the 7 mantissa bits in bits 6..0."""
    w = np.asarray(w, dtype=np.uint16)
    e = ((w >> 7) & 0xFF).astype(np.uint8)
    sm = (((w >> 15) << 7) | (w & 0x7F)).astype(np.uint8)
    return e, sm


def merge_fields(e, sm):
    """Inverse of split_fields: BF16 = sign<<15 | e<<7 | mantissa."""
    e = np.asarray(e, dtype=np.uint16)
    sm = np.asarray(sm, dtype=np.uint16)
    return (((sm >> 7) << 15) | (e << 7) | (sm & 0x7F)).astype(np.uint16)


# ----------------------------------------------------------------------------------------
# Histogram and top-16 palette (exponent-distribution paragraph; R3)
# ----------------------------------------------------------------------------------------
def exponent_histogram(e):
    """Count of each of the 256 exponent values over the whole matrix."""
    return np.bincount(np.asarray(e, np.uint8).ravel(), minlength=256).astype(np.int64)


def palette_from_exponents(exps):
    """A palette given by its caller (the boundary's encode option): the listed exponents,
    which must be 1..16 distinct values 0..255 in ascending order; index = list position."""
    exps = [int(v) for v in exps]
    if not 1 <= len(exps) <= PALETTE_SIZE or any(not 0 <= v <= 255 for v in exps):
        raise ValueError("a palette holds 1..16 exponents in 0..255")
    if any(b <= a for a, b in zip(exps, exps[1:])):
        raise ValueError("palette exponents must be strictly ascending")
    index_of = np.full(256, NONE, dtype=np.uint8)
    for i, x in enumerate(exps):
        index_of[x] = i
    return np.array(exps, dtype=np.uint8), index_of


def build_palette(hist):
    """Top-16 exponents by count (ties: smaller exponent first), listed in ascending
    exponent order (R3).  Returns (palette uint8[n_pal], index_of uint8[256])."""
    present = [x for x in range(256) if hist[x] > 0]
    present.sort(key=lambda x: (-int(hist[x]), x))
    chosen = sorted(present[:PALETTE_SIZE])
    index_of = np.full(256, NONE, dtype=np.uint8)
    for i, x in enumerate(chosen):
        index_of[x] = i
    return np.array(chosen, dtype=np.uint8), index_of


# ----------------------------------------------------------------------------------------
# Shapes and tiled layout (R8)
# ----------------------------------------------------------------------------------------
def padded_rows(n):
    return -(-n // TILE_ROWS) * TILE_ROWS


def check_shape(n, k):
    if n < 1 or k < SEG or k % SEG:
        raise ValueError(f"need n >= 1 and k a positive multiple of {SEG}; got {n}x{k}")


def pad_rows(a, n_pad):
    out = np.zeros((n_pad,) + a.shape[1:], dtype=a.dtype)
    out[: a.shape[0]] = a
    return out


def tile_bytes(a):
    """[Np, K] byte matrix -> flat bytes in sub-tile order:
    offset(n, k) = ((t*(K/16) + k//16)*16 + r)*16 + k%16, with t = n//16, r = n%16."""
    n_pad, k = a.shape
    t = n_pad // TILE_ROWS
    return a.reshape(t, TILE_ROWS, k // KSUB, KSUB).transpose(0, 2, 1, 3).reshape(-1).copy()


def untile_bytes(flat, n_pad, k):
    t = n_pad // TILE_ROWS
    return flat.reshape(t, k // KSUB, TILE_ROWS, KSUB).transpose(0, 2, 1, 3).reshape(n_pad, k).copy()


def nibble_shift(i):
    """Bit position of the i-th (0..7) index of an 8-index group inside its 32-bit word:
    even positions fill the low half-word, odd positions the high half-word, so the two
    indices of a BF16 pair sit 16 bits apart (R8)."""
    return 4 * (i >> 1) + 16 * (i & 1)


def pack_indices(idx):
    """[Np, K] palette indices (0..15) -> bytes of the 4-bit index stream.

    Row r of sub-tile (t, j) owns 8 bytes at ((t*(K/16) + j)*16 + r)*8: two little-endian
    u32 words; word w holds columns 16j + 8w + i (i = 0..7) at bit nibble_shift(i)."""
    n_pad, k = idx.shape
    t = n_pad // TILE_ROWS
    g = idx.astype(np.uint32).reshape(t, TILE_ROWS, k // KSUB, 2, 8).transpose(0, 2, 1, 3, 4)
    shifts = np.array([nibble_shift(i) for i in range(8)], dtype=np.uint32)
    words = (g << shifts).sum(axis=-1, dtype=np.uint64).astype(np.uint32)   # disjoint bits
    return words.reshape(-1).astype("<u4").view(np.uint8).copy()


def unpack_indices(buf, n_pad, k):
    t = n_pad // TILE_ROWS
    words = np.frombuffer(np.ascontiguousarray(buf).tobytes(), dtype="<u4").reshape(t, k // KSUB, TILE_ROWS, 2)
    shifts = np.array([nibble_shift(i) for i in range(8)], dtype=np.uint32)
    nib = (words[..., None] >> shifts) & 0xF                       # [t, j, r, w, i]
    return nib.transpose(0, 2, 1, 3, 4).reshape(n_pad, k).astype(np.uint8)


def segment_order(a3):
    """[Np, KB, X] (row, block, ...) -> [T, KB, 16, X]: segments in (tile, block, row) order."""
    n_pad, kb = a3.shape[:2]
    return a3.reshape(n_pad // TILE_ROWS, TILE_ROWS, kb, *a3.shape[2:]).swapaxes(1, 2)


# ----------------------------------------------------------------------------------------
# Verbatim segments (rare-exponent paragraph; R1, R2)
# ----------------------------------------------------------------------------------------
def verbatim_segments(e, index_of):
    """bool [N, K/64]: True where the segment holds an exponent outside the palette."""
    n, k = e.shape
    outside = index_of[e] == NONE
    return outside.reshape(n, k // SEG, SEG).any(axis=2)


def tile_flags(verb, n):
    """uint16 [T, KB]: bit r of flags[t, b] is set when segment (16t + r, b) is verbatim."""
    n_pad = padded_rows(n)
    v = pad_rows(verb, n_pad)
    vt = segment_order(v[:, :, None])[..., 0]                      # [T, KB, 16]
    bits = (1 << np.arange(TILE_ROWS, dtype=np.uint32))
    return (vt.astype(np.uint32) * bits).sum(axis=2, dtype=np.uint32).astype(np.uint16)


# ----------------------------------------------------------------------------------------
# Length-limited Huffman code (Huffman paragraph; R4, R5)
# ----------------------------------------------------------------------------------------
def package_merge_lengths(freqs, lmax=LMAX):
    """Optimal prefix-code lengths with every length <= lmax (package-merge, Larmore and
    Hirschberg 1990).

    Leaves are sorted by (weight, symbol).  lmax-1 times: pair up neighbours of the current
    list into packages (an odd last item is dropped) and merge the packages with the leaves
    by weight, a leaf going first on equal weight.  The first 2(n-1) items of the final
    list are kept; a symbol's length is the number of kept items that contain it.
    n = 1 gives length 1; symbols with zero frequency get length 0."""
    freqs = [int(f) for f in freqs]
    syms = [s for s, f in enumerate(freqs) if f > 0]
    lengths = [0] * len(freqs)
    if not syms:
        return lengths
    if len(syms) == 1:
        lengths[syms[0]] = 1
        return lengths
    if len(syms) > (1 << lmax):
        raise ValueError("too many symbols for the length limit")
    leaves = [(freqs[s], (s,)) for s in sorted(syms, key=lambda s: (freqs[s], s))]
    current = list(leaves)
    for _ in range(lmax - 1):
        packages = [(current[2 * i][0] + current[2 * i + 1][0], current[2 * i][1] + current[2 * i + 1][1])
                    for i in range(len(current) // 2)]
        merged, i, j = [], 0, 0
        while i < len(leaves) or j < len(packages):
            if j == len(packages) or (i < len(leaves) and leaves[i][0] <= packages[j][0]):
                merged.append(leaves[i])
                i += 1
            else:
                merged.append(packages[j])
                j += 1
        current = merged
    for _, members in current[: 2 * (len(syms) - 1)]:
        for s in members:
            lengths[s] += 1
    return lengths


def canonical_codes(lengths):
    """Canonical prefix codes: symbols ordered by (length, symbol); the first gets 0, each
    next gets (previous + 1) << (its length - previous length)."""
    order = sorted((s for s, L in enumerate(lengths) if L > 0), key=lambda s: (lengths[s], s))
    codes = [0] * len(lengths)
    code, prev = 0, None
    for s in order:
        if prev is not None:
            code = (code + 1) << (lengths[s] - prev)
        codes[s] = code
        prev = lengths[s]
    return codes


# ----------------------------------------------------------------------------------------
# Bitstream (R6, R7)
# ----------------------------------------------------------------------------------------
def pack_bitstream(symbols, lengths, codes):
    """Concatenate the codes of `symbols` MSB-first into u32 words (stream bit b is bit
    31 - b%32 of word b//32).  Returns (words uint32, start bit of each symbol, total bits).
    Two zero words follow the last stream word."""
    symbols = np.asarray(symbols, dtype=np.int64)
    L = np.asarray(lengths, dtype=np.int64)[symbols]
    C = np.asarray(codes, dtype=np.int64)[symbols]
    ends = np.cumsum(L)
    starts = ends - L
    total = int(ends[-1]) if len(L) else 0
    n_words = (total + 31) // 32 + 2
    w0 = starts >> 5
    room = 32 - (starts & 31) - L                  # < 0: the code spills into the next word
    first = np.where(room >= 0, C << np.maximum(room, 0), C >> np.maximum(-room, 0))
    second = np.where(room < 0, (C << np.minimum(32 + room, 32)) & 0xFFFFFFFF, 0)
    # codes occupy disjoint bits, so adding the pieces of a word equals OR-ing them; every
    # partial sum stays below 2**32 and is exact in float64.
    acc = np.bincount(w0, weights=first.astype(np.float64), minlength=n_words)
    acc += np.bincount(w0 + 1, weights=second.astype(np.float64), minlength=n_words)[:n_words]
    return acc.astype(np.uint64).astype(np.uint32), starts, total


def pack_bitstream_plain(symbols, lengths, codes):
    """Same stream as pack_bitstream, built from a '0'/'1' string (small inputs only)."""
    bits = "".join(format(codes[s], "0%db" % lengths[s]) for s in symbols)
    total = len(bits)
    n_words = (total + 31) // 32 + 2
    bits = bits + "0" * (32 * n_words - total)
    words = np.array([int(bits[32 * i: 32 * i + 32], 2) for i in range(n_words)], dtype=np.uint32)
    return words, total


# ----------------------------------------------------------------------------------------
# Encoder
# ----------------------------------------------------------------------------------------
def analyse(w, n, k, palette=None):
    """Everything the encoder derives from W, as named arrays (no serialisation).

    palette: None builds W's own top-16 (exponent-distribution paragraph); a list of
    ascending exponents replaces that one step (reading R15: a caller-supplied palette, e.g.
    shared by several matrices).  Every later step is unchanged: segments holding an exponent
    outside the palette are verbatim, and the code is built over the other segments' indices."""
    check_shape(n, k)
    w = np.asarray(w, dtype=np.uint16).reshape(n, k)
    e, sm = split_fields(w)
    hist = exponent_histogram(e)
    palette, index_of = build_palette(hist) if palette is None else palette_from_exponents(palette)
    verb = verbatim_segments(e, index_of)
    n_pad = padded_rows(n)
    kb = k // SEG
    T = n_pad // TILE_ROWS
    flags = tile_flags(verb, n)                                    # [T, KB]
    real = segment_order(pad_rows(np.ones((n, kb), bool), n_pad)[:, :, None])[..., 0]   # [T,KB,16]
    verb_t = segment_order(pad_rows(verb, n_pad)[:, :, None])[..., 0]
    coded = real & ~verb_t
    e_seg = segment_order(pad_rows(e, n_pad).reshape(n_pad, kb, SEG))       # [T,KB,16,64]
    vexp = e_seg[verb_t].reshape(-1).copy()
    per_tile_verb = verb_t.reshape(T, -1).sum(axis=1)
    vprefix = np.concatenate([[0], np.cumsum(per_tile_verb)]).astype(np.uint32)
    idx = index_of[pad_rows(e, n_pad)]                               # NONE outside palette
    idx_seg = segment_order(idx.reshape(n_pad, kb, SEG))
    symbols = idx_seg[coded].reshape(-1).astype(np.int64)            # (t, b, r, i) order
    freqs = np.bincount(symbols, minlength=PALETTE_SIZE)[:PALETTE_SIZE] if len(symbols) else np.zeros(16, np.int64)
    return dict(n=n, k=k, e=e, sm=sm, hist=hist, palette=palette, index_of=index_of, verb=verb,
                flags=flags, vprefix=vprefix, vexp=vexp, coded=coded, symbols=symbols, freqs=freqs,
                coded_per_block=coded.sum(axis=2))


def chunk_starts(coded_per_block, chunk):
    """Symbol index of every chunk start and the first chunk of each tile (cbase, T+1
    entries).  coded_per_block [T, KB]: coded segments of each (tile, block).  Chunks
    restart at every block of every tile (R7): block (t, b) with c coded segments holds
    ceil(64 c / S) chunks, all of S symbols but the last."""
    starts, cbase, base = [], [0], 0
    for tile in coded_per_block:
        nch_tile = 0
        for segs in tile:
            nsym = int(segs) * SEG
            nch = -(-nsym // chunk)
            starts.extend(base + c * chunk for c in range(nch))
            nch_tile += nch
            base += nsym
        cbase.append(cbase[-1] + nch_tile)
    return np.array(starts, dtype=np.int64), np.array(cbase, dtype=np.uint32)


def encode(w, n, k, chunk=DEFAULT_CHUNK, lmax=LMAX, palette=None):
    """W (uint16 BF16 bits, [n, k]) -> dict with every section of the format.
    palette: None (W's own top-16) or the caller's ascending exponents (see analyse)."""
    if chunk % SEG or chunk <= 0:
        raise ValueError("chunk must be a positive multiple of 64")
    a = analyse(w, n, k, palette)
    lengths = package_merge_lengths(list(a["freqs"]) + [0] * (PALETTE_SIZE - len(a["freqs"])), lmax)
    codes = canonical_codes(lengths)
    words, sym_start, total = pack_bitstream(a["symbols"], lengths, codes)
    if total >= 1 << 32:
        raise ValueError("stream longer than 2**32 bits")
    cstart, cbase = chunk_starts(a["coded_per_block"], chunk)
    off = np.concatenate([sym_start[cstart], [total]]).astype(np.uint32) if len(cstart) else np.array([total], np.uint32)
    n_pad = padded_rows(n)
    sm_t = tile_bytes(pad_rows(a["sm"], n_pad))
    return dict(n=n, k=k, chunk=chunk, lmax=lmax, palette=a["palette"], lengths=lengths, codes=codes,
                n_verb=int(a["vprefix"][-1]), n_coded=int(len(a["symbols"])), total_bits=total,
                sm=sm_t, flags=a["flags"], vprefix=a["vprefix"], vexp=a["vexp"], cbase=cbase,
                off=off, words=words, freqs=a["freqs"])


# ----------------------------------------------------------------------------------------
# Blob serialisation: 256-byte header, then 256-byte aligned sections
# ----------------------------------------------------------------------------------------
def _section_bytes(enc):
    return [np.ascontiguousarray(enc["sm"], np.uint8).tobytes(),
            np.ascontiguousarray(enc["flags"], "<u2").tobytes(),
            np.ascontiguousarray(enc["vprefix"], "<u4").tobytes(),
            np.ascontiguousarray(enc["vexp"], np.uint8).tobytes(),
            np.ascontiguousarray(enc["cbase"], "<u4").tobytes(),
            np.ascontiguousarray(enc["off"], "<u4").tobytes(),
            np.ascontiguousarray(enc["words"], "<u4").tobytes()]


def serialize(enc):
    """Header layout (little-endian):
      0 magic 'UW1\\0' | 4 version | 8 n | 12 k | 16 tile rows (16) | 20 segment (64)
      24 chunk S | 28 lmax | 32 n_pal | 36 n_verb | 40 n_coded (u64) | 48 total_bits (u64)
      56 n_chunks | 60 n_words | 64 palette[16] | 80 code length[16] | 96 code[16] (u16)
      128 seven (offset u64, size u64) pairs: sm, flags, vprefix, vexp, cbase, off, words
      240..255 zero."""
    secs = _section_bytes(enc)
    pal = np.zeros(16, np.uint8)
    pal[: len(enc["palette"])] = enc["palette"]
    head = bytearray(HEADER_BYTES)
    struct.pack_into("<4sIIIIIIIII", head, 0, MAGIC, VERSION, enc["n"], enc["k"], TILE_ROWS, SEG,
                     enc["chunk"], enc["lmax"], len(enc["palette"]), enc["n_verb"])
    struct.pack_into("<QQII", head, 40, enc["n_coded"], enc["total_bits"], len(enc["off"]) - 1, len(enc["words"]))
    head[64:80] = pal.tobytes()
    head[80:96] = bytes(enc["lengths"])
    struct.pack_into("<16H", head, 96, *enc["codes"])
    pos, table = HEADER_BYTES, []
    for s in secs:
        table.append((pos, len(s)))
        pos += -(-len(s) // ALIGN) * ALIGN
    for i, (o, sz) in enumerate(table):
        struct.pack_into("<QQ", head, 128 + 16 * i, o, sz)
    out = bytearray(pos)
    out[:HEADER_BYTES] = head
    for (o, sz), s in zip(table, secs):
        out[o: o + sz] = s
    return bytes(out)


def parse(blob):
    """Blob bytes -> dict of header fields and section arrays (validates bounds)."""
    blob = bytes(blob)
    if len(blob) < HEADER_BYTES or blob[:4] != MAGIC:
        raise ValueError("bad magic")
    (_, ver, n, k, tr, seg, chunk, lmax, n_pal, n_verb) = struct.unpack_from("<4sIIIIIIIII", blob, 0)
    if ver != VERSION or tr != TILE_ROWS or seg != SEG:
        raise ValueError("unsupported version or geometry")
    n_coded, total_bits, n_chunks, n_words = struct.unpack_from("<QQII", blob, 40)
    d = dict(n=n, k=k, chunk=chunk, lmax=lmax, n_pal=n_pal, n_verb=n_verb, n_coded=n_coded,
             total_bits=total_bits, n_chunks=n_chunks, n_words=n_words,
             palette=np.frombuffer(blob, np.uint8, n_pal, 64).copy(),
             lengths=list(blob[80:96]), codes=list(struct.unpack_from("<16H", blob, 96)))
    if not 1 <= lmax <= LMAX_FORMAT or max(d["lengths"]) > lmax:
        raise ValueError("code lengths above the limit")
    dtypes = dict(sm=np.uint8, flags="<u2", vprefix="<u4", vexp=np.uint8, cbase="<u4", off="<u4", words="<u4")
    for i, name in enumerate(SECTION_NAMES):
        o, sz = struct.unpack_from("<QQ", blob, 128 + 16 * i)
        if o + sz > len(blob):
            raise ValueError("section %s out of bounds" % name)
        d[name] = np.frombuffer(blob, dtypes[name], sz // np.dtype(dtypes[name]).itemsize, o).copy()
    return d


# ----------------------------------------------------------------------------------------
# Decoders
# ----------------------------------------------------------------------------------------
def canonical_decode_tables(lengths):
    """Textbook canonical decoding tables: count[L], first code of length L, position in
    (length, symbol) order of the first symbol of length L."""
    count = [0] * (LMAX_FORMAT + 2)
    for L in lengths:
        if L:
            count[L] += 1
    order = sorted((s for s, L in enumerate(lengths) if L > 0), key=lambda s: (lengths[s], s))
    first, first_pos = [0] * (LMAX_FORMAT + 2), [0] * (LMAX_FORMAT + 2)
    code, pos = 0, 0
    for L in range(1, LMAX_FORMAT + 1):
        code = (code + count[L - 1]) << 1 if L > 1 else 0
        first[L], first_pos[L] = code, pos
        pos += count[L]
    return count, first, first_pos, order


def decode_sequential(words, n_symbols, lengths, codes):
    """Bit-by-bit decode from bit 0 using a (length, code) -> symbol dictionary.  Small
    inputs only."""
    table = {(L, c): s for s, (L, c) in enumerate(zip(lengths, codes)) if L > 0}
    out, pos = [], 0
    for _ in range(n_symbols):
        code, L = 0, 0
        while True:
            bit = (int(words[pos >> 5]) >> (31 - (pos & 31))) & 1
            pos += 1
            code, L = (code << 1) | bit, L + 1
            if (L, code) in table:
                out.append(table[(L, code)])
                break
            if L > LMAX_FORMAT:
                raise ValueError("invalid code at bit %d" % pos)
    return np.array(out, dtype=np.int64), pos


def decode_chunks(words, off, chunk_len, lengths):
    """Decode every chunk in lockstep (one numpy lane per chunk) with the canonical tables.
    chunk_len[c] = number of symbols in chunk c.  Checks that chunk c ends exactly where
    the next chunk's offset (or the stream end) says.  Returns symbols in chunk order."""
    count, first, first_pos, order = canonical_decode_tables(lengths)
    order = np.array(order + [0], dtype=np.int64)
    words64 = np.asarray(words, dtype=np.uint64)
    nch = len(chunk_len)
    pos = np.asarray(off[:nch], dtype=np.int64).copy()
    steps = int(max(chunk_len)) if nch else 0
    out = np.zeros((nch, max(steps, 1)), dtype=np.int64)
    for step in range(steps):
        act = np.nonzero(chunk_len > step)[0]
        p = pos[act]
        wi = p >> 5
        pair = (words64[wi] << np.uint64(32)) | words64[wi + 1]
        window = ((pair >> (np.uint64(64 - LMAX_FORMAT) - (p & 31).astype(np.uint64))) & np.uint64((1 << LMAX_FORMAT) - 1)).astype(np.int64)
        sym = np.full(len(act), -1, dtype=np.int64)
        ln = np.zeros(len(act), dtype=np.int64)
        for L in range(1, LMAX_FORMAT + 1):
            if count[L] == 0:
                continue
            c = window >> (LMAX_FORMAT - L)
            hit = (sym < 0) & (c >= first[L]) & (c < first[L] + count[L])
            sym[hit] = order[first_pos[L] + c[hit] - first[L]]
            ln[hit] = L
        if (sym < 0).any():
            raise ValueError("invalid code in chunk %d" % act[np.argmax(sym < 0)])
        out[act, step] = sym
        pos[act] = p + ln
    ends = np.concatenate([np.asarray(off[1:nch], np.int64), [int(off[nch])]]) if nch else np.zeros(0, np.int64)
    if nch and not np.array_equal(pos, ends):
        raise ValueError("chunk end does not match the next chunk offset")
    return np.concatenate([out[c, : chunk_len[c]] for c in range(nch)]) if nch else np.zeros(0, np.int64)


def chunk_lengths(d):
    """Symbols per chunk, in chunk order, from the verbatim flags (R7: chunks of S symbols
    restarting at every block of every tile; a block's last chunk holds the rest)."""
    coded, _, _ = _coded_and_verbatim_masks(d)
    lens = []
    for tile in coded.sum(axis=2):
        for segs in tile:
            nsym = int(segs) * SEG
            lens.extend(min(d["chunk"], nsym - c) for c in range(0, nsym, d["chunk"]))
    return np.array(lens, dtype=np.int64)


def _coded_and_verbatim_masks(d):
    n, k = d["n"], d["k"]
    n_pad = padded_rows(n)
    T, kb = n_pad // TILE_ROWS, k // SEG
    flags = d["flags"].reshape(T, kb).astype(np.uint32)
    verb = ((flags[:, :, None] >> np.arange(TILE_ROWS, dtype=np.uint32)) & 1).astype(bool)   # [T,KB,16]
    real = segment_order(pad_rows(np.ones((n, kb), bool), n_pad)[:, :, None])[..., 0]
    return real & ~verb, verb, real


def _from_segment_order(seg, n_pad, k):
    """[T, KB, 16, 64] -> [Np, K]."""
    T = seg.shape[0]
    return seg.swapaxes(1, 2).reshape(n_pad, k)


def decode_symbols(d):
    lens = chunk_lengths(d)
    if len(lens) and int(lens.sum()) != d["n_coded"]:
        raise ValueError("chunk table inconsistent with coded symbol count")
    coded, _, _ = _coded_and_verbatim_masks(d)
    per_tile = [sum(-(-int(c) * SEG // d["chunk"]) for c in tile) for tile in coded.sum(axis=2)]
    if len(lens) != d["n_chunks"] or not np.array_equal(np.diff(d["cbase"].astype(np.int64)), per_tile):
        raise ValueError("chunk table inconsistent with the verbatim flags")
    return decode_chunks(d["words"], d["off"], lens, d["lengths"])


def exponents_from_blob(d, symbols=None):
    """[Np, K] exponent bytes: palette values for coded segments, raw bytes for verbatim
    segments, 0 for padding rows."""
    n, k = d["n"], d["k"]
    n_pad, kb = padded_rows(n), k // SEG
    if symbols is None:
        symbols = decode_symbols(d)
    coded, verb, _ = _coded_and_verbatim_masks(d)
    seg = np.zeros((n_pad // TILE_ROWS, kb, TILE_ROWS, SEG), dtype=np.uint8)
    seg[coded] = d["palette"][symbols.reshape(-1, SEG)]
    seg[verb] = d["vexp"].reshape(-1, SEG)
    return _from_segment_order(seg, n_pad, k)


def indices_from_blob(d, symbols=None):
    """[Np, K] palette indices: decoded symbol for coded segments, 0 elsewhere (R2)."""
    n, k = d["n"], d["k"]
    n_pad, kb = padded_rows(n), k // SEG
    if symbols is None:
        symbols = decode_symbols(d)
    coded, _, _ = _coded_and_verbatim_masks(d)
    seg = np.zeros((n_pad // TILE_ROWS, kb, TILE_ROWS, SEG), dtype=np.uint8)
    seg[coded] = symbols.reshape(-1, SEG)
    return _from_segment_order(seg, n_pad, k)


def decode_blob(blob):
    """Full decode: blob -> W (uint16 [n, k])."""
    d = parse(blob)
    n, k = d["n"], d["k"]
    n_pad = padded_rows(n)
    e = exponents_from_blob(d)
    sm = untile_bytes(d["sm"], n_pad, k)
    return merge_fields(e, sm)[:n]


def transcode_blob(blob):
    """Direct-palette index stream (bytes) the load-time transcode must produce."""
    d = parse(blob)
    return pack_indices(indices_from_blob(d))


def exponent_stream_blob(blob):
    """Exponent-only stream (tiled bytes) the exponent-only pipeline must produce."""
    d = parse(blob)
    return tile_bytes(exponents_from_blob(d))


def reconstruct_from_palette(sm_tiled, idx_bytes, flags, vprefix, vexp, palette, n, k):
    """Direct-palette reconstruction: e = palette[index] for non-verbatim segments, the raw
    verbatim exponents otherwise; W = sign+mantissa merged with e.  Returns [n, k]."""
    n_pad, kb = padded_rows(n), k // SEG
    T = n_pad // TILE_ROWS
    idx = unpack_indices(idx_bytes, n_pad, k)
    pal16 = np.zeros(16, np.uint8)
    pal16[: len(palette)] = palette
    e = pal16[idx]
    fl = np.asarray(flags).reshape(T, kb).astype(np.uint32)
    verb = ((fl[:, :, None] >> np.arange(TILE_ROWS, dtype=np.uint32)) & 1).astype(bool)
    seg = segment_order(e.reshape(n_pad, kb, SEG)).copy()
    seg[verb] = np.asarray(vexp, np.uint8).reshape(-1, SEG)
    e = _from_segment_order(seg, n_pad, k)
    sm = untile_bytes(np.asarray(sm_tiled, np.uint8), n_pad, k)
    return merge_fields(e, sm)[:n]


# ----------------------------------------------------------------------------------------
# Sizes (bits per weight)
# ----------------------------------------------------------------------------------------
def bundle_bytes(enc):
    """Bytes of the Huffman bundle: header + every section (unpadded)."""
    return HEADER_BYTES + sum(len(s) for s in _section_bytes(enc))


def resident_palette_bytes(enc):
    """Bytes the direct-palette matmul reads for W: sign+mantissa + 4-bit indices + flags +
    per-tile verbatim prefix + verbatim exponents."""
    n_pad = padded_rows(enc["n"])
    return (n_pad * enc["k"] + n_pad * enc["k"] // 2 + 2 * enc["flags"].size
            + 4 * enc["vprefix"].size + enc["vexp"].size)
