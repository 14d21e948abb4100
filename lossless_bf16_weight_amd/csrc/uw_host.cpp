// libuw host side: the encoder (exponent histogram, top-16 palette, verbatim segments,
// length-limited Huffman code, chunked bitstream), blob validation, error reporting and the
// autotune table.
//
// Method: Cloudflare blog post "Unweight" -- BF16 anatomy, exponent-distribution, Huffman and
// rare-exponent paragraphs (what is stored), four-pipeline paragraphs (what the stream must
// allow: parallel decode to exponents, indices or BF16), autotuning paragraphs (the table).
// The encoder runs at packaging time, so it is multi-threaded host C++: its cost is one pass
// over the BF16 matrix.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

#include "uw_internal.h"

namespace uw {

static thread_local char g_err[512];

uw_status fail(uw_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
void clear_error() { g_err[0] = 0; }

// ---------------------------------------------------------------------------------------
// Small parallel-for over [0, n) in contiguous ranges.
// ---------------------------------------------------------------------------------------
static int worker_count(int64_t work_items) {
  int hw = (int)std::thread::hardware_concurrency();
  if (hw <= 0) hw = 1;
  if (const char* env = getenv("UW_HOST_THREADS")) hw = std::max(1, atoi(env));
  hw = std::min(hw, 64);
  return (int)std::max<int64_t>(1, std::min<int64_t>(hw, work_items));
}

template <class F>
static void parallel_ranges(int64_t n, int nthreads, F&& fn) {
  if (nthreads <= 1 || n <= 1) {
    fn(0, n, 0);
    return;
  }
  std::vector<std::thread> th;
  for (int i = 0; i < nthreads; ++i) {
    int64_t b = n * i / nthreads, e = n * (i + 1) / nthreads;
    th.emplace_back([&fn, b, e, i] { fn(b, e, i); });
  }
  for (auto& t : th) t.join();
}

// ---------------------------------------------------------------------------------------
// Huffman code construction (Huffman paragraph): package-merge with a 12-bit limit, so that
// every code fits the decoder's 2^12-entry lookup table (16 KB: the size the SM-split
// paragraph gives the decode kernel's table).  Blobs may hold codes up to kLmax = 13 bits;
// the decoders take those too (the row decoder through a few secondary table entries).
// Tie rules: leaves ordered by (weight, symbol); when merging, a leaf precedes a package of
// equal weight; a trailing odd item is dropped when packaging.
// ---------------------------------------------------------------------------------------
constexpr int kLmaxEncode = 12;

struct PMItem {
  uint64_t w;
  uint8_t cnt[16];  // how many times each symbol occurs inside this item
};

static void package_merge(const uint64_t freq[16], int lmax, uint8_t len[16]) {
  std::memset(len, 0, 16);
  int syms[16], ns = 0;
  for (int s = 0; s < 16; ++s)
    if (freq[s]) syms[ns++] = s;
  if (ns == 0) return;
  if (ns == 1) {
    len[syms[0]] = 1;
    return;
  }
  std::sort(syms, syms + ns, [&](int a, int b) {
    return freq[a] != freq[b] ? freq[a] < freq[b] : a < b;
  });
  std::vector<PMItem> leaves(ns), cur, pk, merged;
  for (int i = 0; i < ns; ++i) {
    leaves[i].w = freq[syms[i]];
    std::memset(leaves[i].cnt, 0, 16);
    leaves[i].cnt[syms[i]] = 1;
  }
  cur = leaves;
  for (int it = 0; it < lmax - 1; ++it) {
    pk.clear();
    for (size_t i = 0; i + 1 < cur.size(); i += 2) {
      PMItem p;
      p.w = cur[i].w + cur[i + 1].w;
      for (int s = 0; s < 16; ++s) p.cnt[s] = (uint8_t)(cur[i].cnt[s] + cur[i + 1].cnt[s]);
      pk.push_back(p);
    }
    merged.clear();
    size_t i = 0, j = 0;
    while (i < leaves.size() || j < pk.size()) {
      if (j == pk.size() || (i < leaves.size() && leaves[i].w <= pk[j].w))
        merged.push_back(leaves[i++]);
      else
        merged.push_back(pk[j++]);
    }
    cur.swap(merged);
  }
  for (int i = 0; i < 2 * (ns - 1); ++i)
    for (int s = 0; s < 16; ++s) len[s] = (uint8_t)(len[s] + cur[i].cnt[s]);
}

void canonical_codes(const uint8_t len[16], uint16_t code[16]) {
  int order[16], no = 0;
  for (int s = 0; s < 16; ++s)
    if (len[s]) order[no++] = s;
  std::sort(order, order + no, [&](int a, int b) { return len[a] != len[b] ? len[a] < len[b] : a < b; });
  std::memset(code, 0, 32);
  uint32_t c = 0;
  for (int i = 0; i < no; ++i) {
    if (i) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
    code[order[i]] = (uint16_t)c;
  }
}

// ---------------------------------------------------------------------------------------
// Palette (exponent-distribution paragraph): top-16 by count, ties to the smaller exponent,
// listed in ascending exponent order.
// ---------------------------------------------------------------------------------------
static void histogram(const uint16_t* w, int64_t n, int64_t k, uint64_t hist[256]) {
  const int64_t total = n * k;
  int nt = worker_count(total / (1 << 20) + 1);
  std::vector<std::vector<uint64_t>> part(nt, std::vector<uint64_t>(256, 0));
  parallel_ranges(total, nt, [&](int64_t b, int64_t e, int tid) {
    uint64_t* h = part[tid].data();
    for (int64_t i = b; i < e; ++i) h[(w[i] >> 7) & 0xFF]++;
  });
  for (int x = 0; x < 256; ++x) {
    hist[x] = 0;
    for (int t = 0; t < nt; ++t) hist[x] += part[t][x];
  }
}

static void palette_from_hist(const uint64_t hist[256], uw_palette* p) {
  int cand[256], nc = 0;
  for (int x = 0; x < 256; ++x)
    if (hist[x]) cand[nc++] = x;
  std::stable_sort(cand, cand + nc, [&](int a, int b) { return hist[a] != hist[b] ? hist[a] > hist[b] : a < b; });
  int np = std::min(nc, 16);
  std::sort(cand, cand + np);
  p->n = (uint32_t)np;
  std::memset(p->exp, 0, 16);
  std::memset(p->index_of, 0xFF, 256);
  for (int i = 0; i < np; ++i) {
    p->exp[i] = (uint8_t)cand[i];
    p->index_of[cand[i]] = (uint8_t)i;
  }
  for (int x = 0; x < 256; ++x) p->hist[x] = hist[x];
}

// A caller palette (uw_encode's p): size 1..16, exponents strictly ascending, index_of the
// exact inverse of exp (0xFF for every exponent outside it).
static uw_status check_palette(const uw_palette* p) {
  if (p->n < 1 || p->n > 16) return fail(UW_E_ARG, "palette size %u is not in 1..16", p->n);
  for (uint32_t i = 1; i < p->n; ++i)
    if (p->exp[i] <= p->exp[i - 1]) return fail(UW_E_ARG, "palette exponents are not strictly ascending");
  uint8_t inv[256];
  std::memset(inv, 0xFF, 256);
  for (uint32_t i = 0; i < p->n; ++i) inv[p->exp[i]] = (uint8_t)i;
  for (int x = 0; x < 256; ++x)
    if (p->index_of[x] != inv[x]) return fail(UW_E_ARG, "palette index_of[%d] = %u, expected %u", x, p->index_of[x], inv[x]);
  return UW_OK;
}

static uw_status check_shape(int64_t n, int64_t k) {
  if (n < 1 || k < kSeg) return fail(UW_E_ARG, "n=%lld k=%lld must be positive (k >= 64)", (long long)n, (long long)k);
  if (k % kSeg) return fail(UW_E_SHAPE, "k=%lld is not a multiple of 64", (long long)k);
  if (k > kMaxK) return fail(UW_E_SHAPE, "k=%lld exceeds %lld", (long long)k, (long long)kMaxK);
  if (n > (int64_t)1 << 24) return fail(UW_E_SHAPE, "n=%lld exceeds 2^24", (long long)n);
  return UW_OK;
}

// ---------------------------------------------------------------------------------------
// Encoder state and passes
// ---------------------------------------------------------------------------------------
struct Layout {
  int64_t n, k, np, T, kb;
  int32_t chunk;
  uint64_t sec_size[kNumSections], sec_off[kNumSections], total;
};

static void layout_sections(Layout& L, uint64_t n_verb, uint64_t n_chunks, uint64_t n_words) {
  L.sec_size[SEC_SM] = (uint64_t)L.np * L.k;
  L.sec_size[SEC_FLAGS] = 2ull * L.T * L.kb;
  L.sec_size[SEC_VPREFIX] = 4ull * (L.T + 1);
  L.sec_size[SEC_VEXP] = 64ull * n_verb;
  L.sec_size[SEC_CBASE] = 4ull * (L.T + 1);
  L.sec_size[SEC_OFF] = 4ull * (n_chunks + 1);
  L.sec_size[SEC_WORDS] = 4ull * n_words;
  uint64_t pos = kHeaderBytes;
  for (int s = 0; s < kNumSections; ++s) {
    L.sec_off[s] = pos;
    pos += align_up(L.sec_size[s], kAlign);
  }
  L.total = pos;
}

// Bit writer over a shared word array: interior words of a thread's range are stored, the
// first and last words it touches are OR-ed in after all threads finish (shared with the
// neighbouring ranges).
struct BitWriter {
  uint32_t* words;
  uint64_t acc = 0;
  int nacc = 0;
  uint64_t next_word = 0;
  uint64_t first_word = 0;
  bool first_pending = true;
  uint32_t first_val = 0, last_val = 0;
  uint64_t last_word = UINT64_MAX;
  uint64_t pos = 0;  // absolute bit position

  void start(uint32_t* w, uint64_t bit0) {
    words = w;
    pos = bit0;
    next_word = first_word = bit0 >> 5;
    nacc = (int)(bit0 & 31);
    acc = 0;
  }
  // The first word may be shared with the previous range and the most recent word with the
  // next one: both are held back; every word in between is stored as soon as it is complete.
  inline void emit(uint32_t v) {
    const uint64_t wi = next_word++;
    if (first_pending) {
      first_pending = false;
      first_val = v;
      return;
    }
    if (last_word != UINT64_MAX) words[last_word] = last_val;
    last_word = wi;
    last_val = v;
  }
  inline void put(uint32_t code, int len) {
    acc = (acc << len) | code;
    nacc += len;
    pos += (uint64_t)len;
    if (nacc >= 32) {
      nacc -= 32;
      emit((uint32_t)(acc >> nacc));
      acc &= (nacc ? ((1ull << nacc) - 1) : 0ull);
    }
  }
  void finish() {
    if (nacc > 0) emit((uint32_t)(acc << (32 - nacc)));
  }
};

static int tile_rows(int64_t n, int64_t t) { return (int)std::min<int64_t>(kTileRows, n - t * kTileRows); }

// Non-verbatim real rows of one (tile, block).
static int block_coded_rows(uint32_t flags, int rows) {
  const uint32_t realmask = rows == kTileRows ? 0xFFFFu : ((1u << rows) - 1u);
  return __builtin_popcount(realmask & ~flags);
}

// Chunks of one tile: chunks restart at every 64-column block, so block b holds
// ceil(64 * coded rows of b / chunk) of them.
static uint32_t tile_chunks(const uint16_t* flags, int64_t kb, int rows, int chunk) {
  uint64_t c = 0;
  for (int64_t b = 0; b < kb; ++b) c += ((uint64_t)block_coded_rows(flags[b], rows) * kSeg + chunk - 1) / chunk;
  return (uint32_t)c;
}

static uw_status encode_impl(const uint16_t* w, int64_t n, int64_t k, const uw_palette* p_in, int32_t chunk,
                             uint8_t* blob, size_t cap, size_t* used) {
  uw_status st = check_shape(n, k);
  if (st) return st;
  if (p_in && (st = check_palette(p_in))) return st;
  if (chunk == 0) chunk = kDefaultChunk;
  if (chunk < kSeg || chunk > UW_MAX_CHUNK || chunk % kSeg)
    return fail(UW_E_ARG, "chunk=%d must be a multiple of 64 in [64, %d]", chunk, UW_MAX_CHUNK);

  Layout L;
  L.n = n;
  L.k = k;
  L.np = padded_rows(n);
  L.T = L.np / kTileRows;
  L.kb = k / kSeg;
  L.chunk = chunk;

  uw_palette pal;
  if (p_in) {
    std::memset(&pal, 0, sizeof(pal));
    pal.n = p_in->n;
    for (uint32_t i = 0; i < pal.n; ++i) pal.exp[i] = p_in->exp[i];
    std::memcpy(pal.index_of, p_in->index_of, 256);
  } else {
    uint64_t hist[256];
    histogram(w, n, k, hist);
    palette_from_hist(hist, &pal);
  }
  const uint8_t* index_of = pal.index_of;

  // Pass 1 (per tile): verbatim flags, per-tile symbol counts.
  std::vector<uint16_t> flags((size_t)(L.T * L.kb), 0);
  std::vector<uint64_t> tile_freq((size_t)L.T * 16, 0);
  std::vector<uint32_t> tile_verb((size_t)L.T, 0);
  int nt = worker_count(L.T);
  parallel_ranges(L.T, nt, [&](int64_t t0, int64_t t1, int) {
    for (int64_t t = t0; t < t1; ++t) {
      const int rows = (int)std::min<int64_t>(kTileRows, n - t * kTileRows);
      uint64_t* fr = &tile_freq[(size_t)t * 16];
      uint32_t nv = 0;
      for (int r = 0; r < rows; ++r) {
        const uint16_t* row = w + (size_t)(t * kTileRows + r) * k;
        for (int64_t b = 0; b < L.kb; ++b) {
          const uint16_t* sg = row + b * kSeg;
          bool verb = false;
          for (int i = 0; i < kSeg; ++i) verb |= index_of[(sg[i] >> 7) & 0xFF] == 0xFF;
          if (verb) {
            flags[(size_t)(t * L.kb + b)] |= (uint16_t)(1u << r);
            ++nv;
          } else {
            for (int i = 0; i < kSeg; ++i) fr[index_of[(sg[i] >> 7) & 0xFF]]++;
          }
        }
      }
      tile_verb[(size_t)t] = nv;
    }
  });

  // Code.
  uint64_t freq[16] = {0};
  for (int64_t t = 0; t < L.T; ++t)
    for (int s = 0; s < 16; ++s) freq[s] += tile_freq[(size_t)t * 16 + s];
  uint8_t len[16];
  uint16_t code[16];
  package_merge(freq, kLmaxEncode, len);
  canonical_codes(len, code);

  // Per-tile prefix sums: verbatim segments, bits, chunks.
  std::vector<uint32_t> vprefix((size_t)L.T + 1, 0), cbase((size_t)L.T + 1, 0);
  std::vector<uint64_t> tile_bit0((size_t)L.T + 1, 0), tile_sym0((size_t)L.T + 1, 0);
  for (int64_t t = 0; t < L.T; ++t) {
    uint64_t bits = 0, syms = 0;
    for (int s = 0; s < 16; ++s) {
      bits += tile_freq[(size_t)t * 16 + s] * len[s];
      syms += tile_freq[(size_t)t * 16 + s];
    }
    vprefix[t + 1] = vprefix[t] + tile_verb[t];
    tile_bit0[t + 1] = tile_bit0[t] + bits;
    tile_sym0[t + 1] = tile_sym0[t] + syms;
    cbase[t + 1] = cbase[t] + tile_chunks(flags.data() + t * L.kb, L.kb, tile_rows(n, t), chunk);
  }
  const uint64_t total_bits = tile_bit0[L.T];
  const uint64_t n_coded = tile_sym0[L.T];
  if (total_bits >= (1ull << 32)) return fail(UW_E_SHAPE, "stream of %llu bits exceeds 2^32", (unsigned long long)total_bits);
  const uint64_t n_chunks = cbase[L.T];
  const uint64_t n_words = (total_bits + 31) / 32 + 2;
  const uint64_t n_verb = vprefix[L.T];
  layout_sections(L, n_verb, n_chunks, n_words);
  *used = L.total;
  if (!blob) return UW_OK;
  if (cap < L.total) return fail(UW_E_WORKSPACE, "blob capacity %zu < %llu bytes", cap, (unsigned long long)L.total);

  std::memset(blob, 0, L.total);
  Header* h = reinterpret_cast<Header*>(blob);
  std::memcpy(h->magic, "UW1\0", 4);
  h->version = kVersion;
  h->n = (uint32_t)n;
  h->k = (uint32_t)k;
  h->tile_rows = kTileRows;
  h->seg = kSeg;
  h->chunk = (uint32_t)chunk;
  h->lmax = kLmaxEncode;
  h->n_pal = pal.n;
  h->n_verb = (uint32_t)n_verb;
  h->n_coded = n_coded;
  h->total_bits = total_bits;
  h->n_chunks = (uint32_t)n_chunks;
  h->n_words = (uint32_t)n_words;
  std::memcpy(h->palette, pal.exp, 16);
  std::memcpy(h->code_len, len, 16);
  std::memcpy(h->code, code, 32);
  for (int s = 0; s < kNumSections; ++s) {
    h->sec[s][0] = L.sec_off[s];
    h->sec[s][1] = L.sec_size[s];
  }
  uint8_t* sm_out = blob + L.sec_off[SEC_SM];
  std::memcpy(blob + L.sec_off[SEC_FLAGS], flags.data(), L.sec_size[SEC_FLAGS]);
  std::memcpy(blob + L.sec_off[SEC_VPREFIX], vprefix.data(), L.sec_size[SEC_VPREFIX]);
  std::memcpy(blob + L.sec_off[SEC_CBASE], cbase.data(), L.sec_size[SEC_CBASE]);
  uint8_t* vexp = blob + L.sec_off[SEC_VEXP];
  uint32_t* off = reinterpret_cast<uint32_t*>(blob + L.sec_off[SEC_OFF]);
  uint32_t* words = reinterpret_cast<uint32_t*>(blob + L.sec_off[SEC_WORDS]);
  off[n_chunks] = (uint32_t)total_bits;

  // Pass 2 (per tile range): sign+mantissa sub-tiles, verbatim exponents, bitstream, offsets.
  const int64_t ksub = k / kSub;
  std::vector<BitWriter> writers(nt);
  parallel_ranges(L.T, nt, [&](int64_t t0, int64_t t1, int tid) {
    BitWriter& bw = writers[tid];
    bw.start(words, tile_bit0[t0]);
    for (int64_t t = t0; t < t1; ++t) {
      const int rows = (int)std::min<int64_t>(kTileRows, n - t * kTileRows);
      for (int r = 0; r < rows; ++r) {
        const uint16_t* row = w + (size_t)(t * kTileRows + r) * k;
        for (int64_t c = 0; c < k; ++c) {
          const uint16_t v = row[c];
          sm_out[(((size_t)t * ksub + c / kSub) * kTileRows + r) * kSub + (c % kSub)] =
              (uint8_t)(((v >> 15) << 7) | (v & 0x7F));
        }
      }
      uint64_t vrank = vprefix[t];
      uint64_t chunk_id = cbase[t];
      for (int64_t b = 0; b < L.kb; ++b) {
        const uint16_t f = flags[(size_t)(t * L.kb + b)];
        uint64_t sym = 0;               // coded symbols emitted in this block (chunks restart here)
        for (int r = 0; r < rows; ++r) {
          const uint16_t* sg = w + (size_t)(t * kTileRows + r) * k + b * kSeg;
          if ((f >> r) & 1) {
            uint8_t* dst = vexp + vrank * kSeg;
            for (int i = 0; i < kSeg; ++i) dst[i] = (uint8_t)((sg[i] >> 7) & 0xFF);
            ++vrank;
            continue;
          }
          for (int i = 0; i < kSeg; ++i) {
            if (sym % (uint64_t)chunk == 0) off[chunk_id++] = (uint32_t)bw.pos;
            const int s = index_of[(sg[i] >> 7) & 0xFF];
            bw.put(code[s], len[s]);
            ++sym;
          }
        }
      }
    }
    bw.finish();
  });
  for (int i = 0; i < nt; ++i) {
    BitWriter& bw = writers[i];
    if (!bw.first_pending) words[bw.first_word] |= bw.first_val;
    if (bw.last_word != UINT64_MAX) words[bw.last_word] |= bw.last_val;
  }
  return UW_OK;
}

// ---------------------------------------------------------------------------------------
// Validation (shared by uw_blob_info and uw_dmat_bind)
// ---------------------------------------------------------------------------------------
static int popc16(uint32_t v) { return __builtin_popcount(v & 0xFFFF); }

uw_status validate_blob(const void* blob, size_t bytes, uw_info* info) {
  if (!blob || !info) return fail(UW_E_ARG, "null blob or info");
  if (bytes < (size_t)kHeaderBytes) return fail(UW_E_FORMAT, "blob shorter than its header");
  const Header* h = reinterpret_cast<const Header*>(blob);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(blob);
  if (std::memcmp(h->magic, "UW1\0", 4)) return fail(UW_E_FORMAT, "bad magic");
  if (h->version != kVersion) return fail(UW_E_FORMAT, "unsupported version %u", h->version);
  if (h->tile_rows != kTileRows || h->seg != kSeg) return fail(UW_E_FORMAT, "unsupported tile geometry");
  if (h->n < 1 || h->k < (uint32_t)kSeg || h->k % kSeg || h->k > kMaxK || h->n > (1u << 24))
    return fail(UW_E_FORMAT, "bad shape %u x %u", h->n, h->k);
  if (h->chunk < (uint32_t)kSeg || h->chunk > UW_MAX_CHUNK || h->chunk % kSeg) return fail(UW_E_FORMAT, "bad chunk %u", h->chunk);
  if (h->lmax < 1 || h->lmax > (uint32_t)kLmax) return fail(UW_E_FORMAT, "unsupported code length limit %u", h->lmax);
  if (h->n_pal < 1 || h->n_pal > 16) return fail(UW_E_FORMAT, "bad palette size %u", h->n_pal);
  for (uint32_t i = 1; i < h->n_pal; ++i)
    if (h->palette[i] <= h->palette[i - 1]) return fail(UW_E_FORMAT, "palette not strictly ascending");
  uint64_t kraft = 0;
  int nsym = 0;
  for (int s = 0; s < 16; ++s) {
    if (h->code_len[s] > h->lmax) return fail(UW_E_FORMAT, "code length %u above the limit %u", (unsigned)h->code_len[s], h->lmax);
    if (h->code_len[s] && s >= (int)h->n_pal) return fail(UW_E_FORMAT, "code for a symbol outside the palette");
    if (h->code_len[s]) {
      kraft += 1ull << (kLmax - h->code_len[s]);
      ++nsym;
    }
  }
  if (kraft > (1ull << kLmax)) return fail(UW_E_FORMAT, "code lengths violate Kraft");
  uint16_t canon[16];
  canonical_codes(h->code_len, canon);
  for (int s = 0; s < 16; ++s)
    if (h->code_len[s] && canon[s] != h->code[s]) return fail(UW_E_FORMAT, "codes are not canonical");
  const int64_t n = h->n, k = h->k, np = padded_rows(n), T = np / kTileRows, kb = k / kSeg;
  const uint64_t need_words = (h->total_bits + 31) / 32 + 2;
  if (h->total_bits >= (1ull << 32)) return fail(UW_E_FORMAT, "stream too long");
  if (h->n_words < need_words) return fail(UW_E_FORMAT, "word count too small for the stream");
  if (h->n_coded && nsym == 0) return fail(UW_E_FORMAT, "coded symbols without a code");
  const uint64_t expect[kNumSections] = {(uint64_t)np * k, 2ull * T * kb, 4ull * (T + 1), 64ull * h->n_verb,
                                         4ull * (T + 1), 4ull * ((uint64_t)h->n_chunks + 1), 4ull * h->n_words};
  uint64_t end = kHeaderBytes;
  for (int s = 0; s < kNumSections; ++s) {
    if (h->sec[s][1] != expect[s]) return fail(UW_E_FORMAT, "section %d has %llu bytes, expected %llu", s,
                                                (unsigned long long)h->sec[s][1], (unsigned long long)expect[s]);
    if (h->sec[s][0] % 4 || h->sec[s][0] < end || h->sec[s][0] + h->sec[s][1] > bytes)
      return fail(UW_E_FORMAT, "section %d out of bounds", s);
    end = h->sec[s][0] + h->sec[s][1];
  }
  const uint16_t* flags = reinterpret_cast<const uint16_t*>(base + h->sec[SEC_FLAGS][0]);
  const uint32_t* vprefix = reinterpret_cast<const uint32_t*>(base + h->sec[SEC_VPREFIX][0]);
  const uint32_t* cbase = reinterpret_cast<const uint32_t*>(base + h->sec[SEC_CBASE][0]);
  const uint32_t* off = reinterpret_cast<const uint32_t*>(base + h->sec[SEC_OFF][0]);
  if (vprefix[0] != 0 || cbase[0] != 0) return fail(UW_E_FORMAT, "prefix tables must start at 0");
  uint64_t coded_total = 0;
  for (int64_t t = 0; t < T; ++t) {
    const int rows = (int)std::min<int64_t>(kTileRows, n - t * kTileRows);
    const uint32_t realmask = rows == 16 ? 0xFFFFu : ((1u << rows) - 1);
    uint64_t nv = 0;
    for (int64_t b = 0; b < kb; ++b) {
      const uint32_t f = flags[t * kb + b];
      if (f & ~realmask) return fail(UW_E_FORMAT, "verbatim flag on a padding row");
      nv += (uint64_t)popc16(f);
    }
    if ((uint64_t)vprefix[t + 1] != vprefix[t] + nv) return fail(UW_E_FORMAT, "vprefix inconsistent with flags");
    const uint64_t nsy = ((uint64_t)rows * kb - nv) * kSeg;
    if ((uint64_t)cbase[t + 1] < cbase[t] ||
        (uint64_t)cbase[t + 1] - cbase[t] != tile_chunks(flags + t * kb, kb, rows, (int)h->chunk))
      return fail(UW_E_FORMAT, "cbase inconsistent");
    coded_total += nsy;
  }
  if (vprefix[T] != h->n_verb) return fail(UW_E_FORMAT, "verbatim count mismatch");
  if (cbase[T] != h->n_chunks) return fail(UW_E_FORMAT, "chunk count mismatch");
  if (coded_total != h->n_coded) return fail(UW_E_FORMAT, "coded symbol count mismatch");
  int minlen = 99, maxlen = 0;
  for (int s = 0; s < 16; ++s)
    if (h->code_len[s]) {
      minlen = std::min<int>(minlen, h->code_len[s]);
      maxlen = std::max<int>(maxlen, h->code_len[s]);
    }
  if (off[h->n_chunks] != h->total_bits) return fail(UW_E_FORMAT, "last offset != total bits");
  // Every chunk spans between minlen and maxlen bits per symbol: bounds every decoder read.
  for (int64_t t = 0; t < T; ++t) {
    const int rows = tile_rows(n, t);
    uint32_t c = cbase[t];
    for (int64_t b = 0; b < kb; ++b) {
      const uint64_t nsy = (uint64_t)block_coded_rows(flags[t * kb + b], rows) * kSeg;
      for (uint64_t s0 = 0; s0 < nsy; s0 += h->chunk, ++c) {
        const uint64_t cnt = std::min<uint64_t>(h->chunk, nsy - s0);
        const uint64_t span = (uint64_t)off[c + 1] - off[c];
        if (off[c + 1] < off[c] || span < cnt * minlen || span > cnt * maxlen)
          return fail(UW_E_FORMAT, "chunk %u offsets inconsistent", c);
      }
    }
  }
  if (h->n_chunks && off[0] != 0) return fail(UW_E_FORMAT, "first chunk must start at bit 0");

  std::memset(info, 0, sizeof(*info));
  info->n = n;
  info->k = k;
  info->np = np;
  info->tiles = T;
  info->kb = kb;
  info->chunk = (int32_t)h->chunk;
  info->lmax = (int32_t)h->lmax;
  info->n_pal = (int32_t)h->n_pal;
  info->affine = 1;
  for (uint32_t i = 1; i < h->n_pal; ++i)
    if (h->palette[i] != (uint8_t)(h->palette[0] + i)) info->affine = 0;
  if ((int)h->palette[0] + 15 > 255) info->affine = 0;  // unused indices must stay in range
  info->n_verb = h->n_verb;
  info->n_coded = (int64_t)h->n_coded;
  info->total_bits = (int64_t)h->total_bits;
  info->n_chunks = h->n_chunks;
  info->n_words = h->n_words;
  std::memcpy(info->palette, h->palette, 16);
  std::memcpy(info->code_len, h->code_len, 16);
  std::memcpy(info->code, h->code, 32);
  for (int s = 0; s < kNumSections; ++s) {
    info->sec_off[s] = h->sec[s][0];
    info->sec_size[s] = h->sec[s][1];
  }
  info->blob_bytes = h->sec[SEC_WORDS][0] + align_up(h->sec[SEC_WORDS][1], kAlign);
  info->idx_bytes = (uint64_t)np * k / 2;
  info->resident_bytes = (uint64_t)np * k + info->idx_bytes + expect[SEC_FLAGS] + expect[SEC_VPREFIX] + expect[SEC_VEXP];
  clear_error();
  return UW_OK;
}

// ---------------------------------------------------------------------------------------
// Autotune table
// ---------------------------------------------------------------------------------------
// Two maps: the pipeline UW_PIPE_AUTO takes for (n, k, m), and the variant each concrete
// pipeline (and the uncompressed UW_PIPE_BF16 key) runs with when called with variant -1.
static std::mutex g_tune_mu;
static std::map<std::tuple<int64_t, int64_t, int32_t>, std::pair<int32_t, int32_t>> g_tune;
static std::map<std::tuple<int64_t, int64_t, int32_t, int32_t>, int32_t> g_tune_var;

// Entries are looked up by (n, k, m); a batch size with no entry takes the entry of the nearest
// measured batch size for the same (n, k) (nearest by ratio, the smaller one on a tie), so a
// table measured at a few M covers the sizes in between.
static double m_distance(int32_t a, int32_t b) { return std::fabs(std::log((double)a / (double)b)); }

bool autotune_lookup(int64_t n, int64_t k, int32_t m, int32_t* pipeline, int32_t* variant) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto lo = g_tune.lower_bound(std::make_tuple(n, k, INT32_MIN));
  auto hi = g_tune.upper_bound(std::make_tuple(n, k, INT32_MAX));
  auto best = g_tune.end();
  for (auto it = lo; it != hi; ++it)
    if (best == g_tune.end() || m_distance(std::get<2>(it->first), m) < m_distance(std::get<2>(best->first), m))
      best = it;
  if (best == g_tune.end()) return false;
  *pipeline = best->second.first;
  *variant = best->second.second;
  return true;
}

int32_t autotune_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto lo = g_tune_var.lower_bound(std::make_tuple(n, k, INT32_MIN, INT32_MIN));
  auto hi = g_tune_var.upper_bound(std::make_tuple(n, k, INT32_MAX, INT32_MAX));
  int32_t v = -1, bm = 0;
  for (auto it = lo; it != hi; ++it) {
    if (std::get<3>(it->first) != pipeline) continue;
    const int32_t em = std::get<2>(it->first);
    if (v < 0 || m_distance(em, m) < m_distance(bm, m)) {
      v = it->second;
      bm = em;
    }
  }
  return v;
}

}  // namespace uw

using namespace uw;

extern "C" {

const char* uw_last_error(void) { return g_err; }
int32_t uw_version(void) { return 10000; }

uw_status uw_build_palette(const uint16_t* w, int64_t n, int64_t k, uw_palette* out) {
  if (!w || !out) return fail(UW_E_ARG, "null argument");
  uw_status st = check_shape(n, k);
  if (st) return st;
  uint64_t hist[256];
  histogram(w, n, k, hist);
  palette_from_hist(hist, out);
  clear_error();
  return UW_OK;
}

uw_status uw_encode_bound(int64_t n, int64_t k, int32_t chunk, size_t* bytes) {
  if (!bytes) return fail(UW_E_ARG, "null bytes");
  uw_status st = check_shape(n, k);
  if (st) return st;
  if (chunk == 0) chunk = kDefaultChunk;
  if (chunk < kSeg || chunk > UW_MAX_CHUNK || chunk % kSeg) return fail(UW_E_ARG, "bad chunk %d", chunk);
  Layout L;
  L.n = n;
  L.k = k;
  L.np = padded_rows(n);
  L.T = L.np / kTileRows;
  L.kb = k / kSeg;
  const uint64_t nk = (uint64_t)n * k;
  const uint64_t chunks = (uint64_t)L.T * L.kb * ((kTileRows * kSeg + chunk - 1) / chunk);
  const uint64_t nverb = (uint64_t)n * L.kb;
  layout_sections(L, nverb, chunks, (nk * kLmax + 31) / 32 + 2);
  *bytes = L.total;
  clear_error();
  return UW_OK;
}

uw_status uw_encode(const uint16_t* w, int64_t n, int64_t k, const uw_palette* p, int32_t chunk, void* blob,
                    size_t cap, size_t* used) {
  if (!w || !used) return fail(UW_E_ARG, "null argument");
  try {
    uw_status st = encode_impl(w, n, k, p, chunk, reinterpret_cast<uint8_t*>(blob), cap, used);
    if (st == UW_OK) clear_error();
    return st;
  } catch (const std::bad_alloc&) {
    return fail(UW_E_NOMEM, "host allocation failed");
  }
}

uw_status uw_blob_info(const void* blob_host, size_t bytes, uw_info* out) {
  try {
    return validate_blob(blob_host, bytes, out);
  } catch (const std::bad_alloc&) {
    return fail(UW_E_NOMEM, "host allocation failed");
  }
}

static uw_status check_tune_key(int64_t n, int64_t k, int32_t m, int32_t variant) {
  if (variant < -1 || variant >= uw_variant_count()) return fail(UW_E_ARG, "bad variant %d", variant);
  if (n < 1 || k < 1 || m < 1 || m > UW_MAX_M) return fail(UW_E_ARG, "bad key");
  return UW_OK;
}

uw_status uw_autotune_set(int64_t n, int64_t k, int32_t m, int32_t pipeline, int32_t variant) {
  if (pipeline < UW_PIPE_FULL_DECODE || pipeline > UW_PIPE_DIRECT_PALETTE)
    return fail(UW_E_ARG, "pipeline %d is not a concrete pipeline", pipeline);
  uw_status st = check_tune_key(n, k, m, variant);
  if (st) return st;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune[std::make_tuple(n, k, m)] = std::make_pair(pipeline, variant);
  if (variant >= 0) g_tune_var[std::make_tuple(n, k, m, pipeline)] = variant;
  clear_error();
  return UW_OK;
}

uw_status uw_autotune_set_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline, int32_t variant) {
  if (pipeline < UW_PIPE_FULL_DECODE || pipeline > UW_PIPE_BF16)
    return fail(UW_E_ARG, "pipeline %d has no variant of its own", pipeline);
  uw_status st = check_tune_key(n, k, m, variant);
  if (st) return st;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  if (variant < 0)
    g_tune_var.erase(std::make_tuple(n, k, m, pipeline));
  else
    g_tune_var[std::make_tuple(n, k, m, pipeline)] = variant;
  clear_error();
  return UW_OK;
}

uw_status uw_autotune_get(int64_t n, int64_t k, int32_t m, int32_t* pipeline, int32_t* variant) {
  if (!pipeline || !variant) return fail(UW_E_ARG, "null argument");
  uw_status st = check_tune_key(n, k, m, -1);
  if (st) return st;
  if (!autotune_lookup(n, k, m, pipeline, variant)) {
    *pipeline = UW_PIPE_DIRECT_PALETTE;
    *variant = -1;
  }
  clear_error();
  return UW_OK;
}

uw_status uw_autotune_get_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline, int32_t* variant) {
  if (!variant) return fail(UW_E_ARG, "null argument");
  if (pipeline < UW_PIPE_FULL_DECODE || pipeline > UW_PIPE_BF16)
    return fail(UW_E_ARG, "pipeline %d has no variant of its own", pipeline);
  uw_status st = check_tune_key(n, k, m, -1);
  if (st) return st;
  *variant = autotune_variant(n, k, m, pipeline);
  clear_error();
  return UW_OK;
}

uw_status uw_autotune_clear(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune.clear();
  g_tune_var.clear();
  clear_error();
  return UW_OK;
}

uw_status uw_autotune_load(const char* path) {
  if (!path) return fail(UW_E_ARG, "null path");
  std::ifstream in(path);
  if (!in) return fail(UW_E_ARG, "cannot open %s", path);
  std::string line;
  int lineno = 0;
  // (is_variant_line, n, k, m, pipeline, variant); applied only once the whole file parsed.
  std::vector<std::tuple<bool, int64_t, int64_t, int32_t, int32_t, int32_t>> rows;
  while (std::getline(in, line)) {
    ++lineno;
    const size_t hash = line.find('#');
    if (hash != std::string::npos) line.resize(hash);
    std::istringstream ss(line);
    std::string first;
    if (!(ss >> first)) continue;
    const bool var_line = first == "variant";
    long long n, k;
    int m, p, v;
    if (var_line) {
      if (!(ss >> n)) return fail(UW_E_ARG, "%s:%d: expected 'variant n k m pipeline variant'", path, lineno);
    } else {
      char* end = nullptr;
      n = std::strtoll(first.c_str(), &end, 10);
      if (!end || *end) return fail(UW_E_ARG, "%s:%d: expected 'n k m pipeline variant'", path, lineno);
    }
    std::string rest;
    if (!(ss >> k >> m >> p >> v) || (ss >> rest))
      return fail(UW_E_ARG, "%s:%d: expected 'n k m pipeline variant'", path, lineno);
    rows.emplace_back(var_line, n, k, m, p, v);
  }
  for (auto& r : rows) {
    const int32_t p = std::get<4>(r);
    uw_status st = check_tune_key(std::get<1>(r), std::get<2>(r), std::get<3>(r), std::get<5>(r));
    if (st) return st;
    const int32_t hi = std::get<0>(r) ? UW_PIPE_BF16 : UW_PIPE_DIRECT_PALETTE;
    if (p < UW_PIPE_FULL_DECODE || p > hi) return fail(UW_E_ARG, "%s: pipeline %d not allowed here", path, p);
  }
  for (auto& r : rows) {
    if (std::get<0>(r))
      uw_autotune_set_variant(std::get<1>(r), std::get<2>(r), std::get<3>(r), std::get<4>(r), std::get<5>(r));
    else
      uw_autotune_set(std::get<1>(r), std::get<2>(r), std::get<3>(r), std::get<4>(r), std::get<5>(r));
  }
  clear_error();
  return UW_OK;
}

}  // extern "C"
