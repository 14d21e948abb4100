// Internal definitions shared by the host codec (uw_host.cpp) and the device side
// (uw_device.h and the .hip sources) of libuw.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "uw.h"

namespace uw {

constexpr int kTileRows = 16;     // rows per tile
constexpr int kSeg = 64;          // weights per verbatim segment (one row, along K)
constexpr int kSub = 16;          // columns per sub-tile
constexpr int kLmax = 13;         // maximum Huffman code length
constexpr int kDefaultChunk = 512;
constexpr int kHeaderBytes = 256;
constexpr int kAlign = 256;
constexpr int kNumSections = 7;
constexpr int64_t kMaxK = 65536;  // KB <= 1024 keeps the decoder's per-tile tables small
constexpr uint32_t kVersion = 1;
constexpr int kErrBytes = 256;    // workspace prefix holding the error word

enum Section { SEC_SM = 0, SEC_FLAGS, SEC_VPREFIX, SEC_VEXP, SEC_CBASE, SEC_OFF, SEC_WORDS };

// The 256-byte blob header, field for field.
struct Header {
  char magic[4];
  uint32_t version, n, k, tile_rows, seg, chunk, lmax, n_pal, n_verb;
  uint64_t n_coded, total_bits;
  uint32_t n_chunks, n_words;
  uint8_t palette[16];
  uint8_t code_len[16];
  uint16_t code[16];
  uint64_t sec[kNumSections][2];  // (offset, size) in bytes
  uint8_t reserved[16];
};
static_assert(sizeof(Header) == kHeaderBytes, "header layout");

inline int64_t padded_rows(int64_t n) { return (n + kTileRows - 1) / kTileRows * kTileRows; }
inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Error reporting: both set the thread-local message returned by uw_last_error().
uw_status fail(uw_status st, const char* fmt, ...);
void clear_error();

// Canonical codes from code lengths (symbols ordered by (length, symbol)).
void canonical_codes(const uint8_t len[16], uint16_t code[16]);

// Full host validation of a blob: header, geometry, code, section bounds and the
// consistency of flags/vprefix/cbase/off.  Fills *info.  Returns UW_OK or UW_E_FORMAT.
uw_status validate_blob(const void* blob, size_t bytes, uw_info* info);

}  // namespace uw

// The device view; the caller allocates uw_dmat_size() bytes for it.
struct uw_dmat {
  uint64_t magic;                 // kDmatMagic once bound
  uw_info info;
  const uint8_t* sm;
  const uint16_t* flags;
  const uint32_t* vprefix;
  const uint8_t* vexp;
  const uint32_t* cbase;
  const uint32_t* off;
  const uint32_t* words;
  uint32_t words_cap;             // words readable in the device blob (aligned section)
  uint8_t* idx;                   // direct-palette index stream (caller's), may be null
  int32_t dec_spc, dec_cpb, dec_nb;  // decoder units: segments per chunk, chunks per block, blocks per unit
  uint32_t dec_stage_words;       // most bitstream words one decoder unit stages (16-byte aligned)
};
constexpr uint64_t kDmatMagic = 0x3130544D44575555ull;  // "UUWDMT01"

namespace uw {
// Autotune table (host): lookup for (n, k, m).
bool autotune_lookup(int64_t n, int64_t k, int32_t m, int32_t* pipeline, int32_t* variant);
// Variant recorded for one pipeline (or UW_PIPE_BF16) at (n, k, m); -1 when none.
int32_t autotune_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline);
}  // namespace uw
