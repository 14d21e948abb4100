// libuw Huffman decoder for MI355X (gfx950): chunk-parallel decode of the exponent stream into
// 4-bit palette indices, exponent bytes or BF16 weights.
//
// Method: Cloudflare blog post "Unweight".
//  - Huffman paragraph: the exponent alone is Huffman coded; per-chunk bit offsets let chunks
//    decode in parallel.
//  - SM-split paragraph: the decoder keeps its lookup table in on-chip memory (LDS here).
//  - Four-pipeline paragraphs: decode to BF16 (pipeline 1), to exponent bytes (2), or to 4-bit
//    indices (3, and the load-time transcode of the direct-palette format).
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "uw_device.h"

namespace uw {

// =========================================================================================
// Huffman decoder.
//
// Chunks restart at every 64-column block of every tile, so the work splits into units of
// whole blocks: one workgroup (one wave) per (tile, group of `nb` blocks), lane i decoding one
// chunk of the unit (lane = block-in-unit * cpb + chunk-in-block).  A wave-level prefix sum
// of the blocks' chunk counts places each chunk in the offset table.
//   1. The unit's slice of the bitstream (contiguous: its chunks are consecutive) is staged
//      in LDS with coalesced 16-byte loads, so the serial decode never waits on HBM.
//   2. A 2^10-entry table (LDS) decodes up to four symbols per lookup: entry = four 4-bit
//      symbols (bits 0-15), total length (16-19), first length (20-23), symbol count (29-31).
//      A window whose first code is longer than 10 bits (rare: symbols below 2^-10
//      frequency) has count 0 and points to a block of a secondary table indexed by the next
//      3 bits.  The bit window is two stream words and a funnel-shift amount; the loop body
//      is branch-free apart from the long-code case: the refill word is read every step and
//      used or not, and every step issues a store (to its place when 8 indices are ready,
//      else to an offset out of the buffer's range).  While four or more symbols remain,
//      a lookup takes all the symbols of its entry; the last one to three take one a step.
//   3. Every mode stores each finished 8-index word straight to global memory, in decode
//      order (a lane's words are consecutive, so lines fill from one lane and the L2 does not
//      write partial lines back): the index and exponent modes into the unit's own output
//      range, the BF16 mode into the first 32 bytes a block of the tile's output rows (row q
//      holds the words of each block's q-th coded row).  After a barrier the workgroup reloads
//      its words into LDS (over the table scratch and the stage) and writes every output line
//      once, whole: indices (verbatim and padding rows 0), exponents (verbatim rows raw), or
//      BF16 weights merged with the sign+mantissa bytes.
// =========================================================================================
constexpr int kDecWin = 10;                 // lookup window, bits
constexpr int kDecLut = 1 << kDecWin;       // primary entries
constexpr int kDecSec = 16 * 8;             // secondary entries: 16 blocks of 8 (block 0: invalid)

struct DecArgs {
  const uint32_t* words;
  const uint32_t* off;
  const uint32_t* cbase;
  const uint16_t* flags;
  const uint32_t* vprefix;
  const uint8_t* vexp;
  const uint8_t* sm;
  uint8_t* out;
  uint32_t* err;
  uint32_t words_cap;
  int32_t n, k, kb;
  int32_t spc, cpb, nb;    // coded segments per chunk, max chunks per block, blocks per unit
  uint32_t stage_words;    // LDS words for one unit's bitstream slice (host bound)
  uint32_t tab[4];         // palette, 16 bytes
  uint8_t len[16];
  uint16_t code[16];
  uint32_t pbase;          // first 10-bit prefix of a code longer than 10 bits
  uint32_t pmask;          // bit i: prefix pbase + i starts a long code (its block is i + 1)
  uint32_t sec[kDecSec];   // secondary entries (same format as the primary ones)
};


struct DecLds {            // offsets (bytes) into the dynamic LDS block (the table is static)
  uint32_t image, stage, blk, total;   // image: table-build scratch, then the reloaded words
};
constexpr uint32_t kDecTableBytes = (kDecLut + kDecSec) * 4u;

// stage_words: a multiple of 256 (the bitstream slice is staged in 1 KB DMA steps).  The unit's
// index words come back as 512 bytes a block (index and exponent modes: one run; BF16 mode: at
// most 16 rows of 32 bytes a block, back to back), reloaded in 1 KB steps.
__host__ __device__ inline DecLds dec_lds(int nb, uint32_t stage_words) {
  DecLds L;
  L.image = 0;
  L.stage = kDecLut * 2u;
  L.blk = L.stage + stage_words * 4;
  L.blk = std::max<uint32_t>(L.blk, ((uint32_t)nb * 512u + 1023u) & ~1023u);
  L.total = L.blk + 2u * 64u * 4u;   // block flags, verbatim ranks
  return L;
}

__device__ __forceinline__ uint32_t nibbles_to_index_word(uint32_t v) {
  // Sequential nibbles n0..n7 (n_i at bits 4i) -> index-stream word (even columns in the low
  // half, odd columns in the high half: n_i at bit 4*(i/2) + 16*(i%2)).  Bytes 0 and 2 of px
  // hold (n0 n2) and (n4 n6), those of py (n1 n3) and (n5 n7).
  const uint32_t v4 = v >> 4;
  const uint32_t px = bfi(0x0F0F0F0Fu, v, v4), py = bfi(0x0F0F0F0Fu, v4, v >> 8);
  return perm(py, px, 0x06040200u);
}

__device__ __forceinline__ u32x2 index_word_to_exps(uint32_t iw, const uint32_t tab[4]) {
  // 8 indices of one index-stream word -> 8 exponent bytes in column order.
  const uint32_t e04 = lookup16(iw & 0x0F0F0F0Fu, tab);          // E0 E4 E1 E5
  const uint32_t e26 = lookup16((iw >> 4) & 0x0F0F0F0Fu, tab);   // E2 E6 E3 E7
  return u32x2{perm(e26, e04, 0x06040200u), perm(e26, e04, 0x07050301u)};
}

__device__ __forceinline__ uint32_t bf16_pairs_from(uint32_t s, uint32_t e, int half) {
  // s, e: 4 sign+mantissa bytes and 4 exponent bytes; half 0 -> weights 0,1; 1 -> 2,3.
  const uint32_t sp = perm(s, s, half ? 0x03030202u : 0x01010000u);
  const uint32_t ep = perm(e, e, half ? 0x0C030C02u : 0x0C010C00u) << 7;
  return (sp & 0x807F807Fu) | ep;
}

// Build the multi-symbol table.  tmp (kDecLut u16): first-symbol table, entry = symbol |
// length << 4 | 0x100 for every window whose first code has length <= kDecWin.
__device__ void build_dec_lut(const DecArgs& a, uint32_t* lut, uint16_t* tmp, int lane) {
  for (int i = lane; i < kDecLut / 2; i += 64) reinterpret_cast<uint32_t*>(tmp)[i] = 0;
  __syncthreads();
  for (int s = 0; s < 16; ++s) {
    const int L = a.len[s];
    if (L == 0 || L > kDecWin) continue;
    const uint32_t lo = (uint32_t)a.code[s] << (kDecWin - L), cnt = 1u << (kDecWin - L);
    for (uint32_t i = lane; i < cnt; i += 64) tmp[lo + i] = (uint16_t)(s | (L << 4) | 0x100);
  }
  __syncthreads();
#pragma unroll 4
  for (int w = lane; w < kDecLut; w += 64) {
    const uint32_t e0 = tmp[w];
    uint32_t entry = 0;
    if (e0 & 0x100u) {
      const uint32_t l0 = (e0 >> 4) & 15u;
      uint32_t used = l0, n = 1, syms = e0 & 15u;
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        const uint32_t ej = tmp[(w << used) & (kDecLut - 1)];
        const uint32_t lj = (ej >> 4) & 15u;
        const bool ok = (n == (uint32_t)j) && (ej & 0x100u) && used + lj <= (uint32_t)kDecWin;
        syms |= ok ? (ej & 15u) << (4 * j) : 0u;
        used += ok ? lj : 0u;
        n += ok ? 1u : 0u;
      }
      entry = (n << 29) | (l0 << 20) | (used << 16) | syms;
    } else {
      const uint32_t i = (uint32_t)w - a.pbase;                // long code: secondary block i + 1
      entry = (i < 15u && ((a.pmask >> i) & 1u)) ? i + 1u : 0u;
    }
    lut[w] = entry;
  }
  for (int i = lane; i < kDecSec; i += 64) lut[kDecLut + i] = a.sec[i];
  __syncthreads();
}

template <int MODE>
__global__ __launch_bounds__(64) void k_decode(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsh[];
  constexpr bool kDirect = MODE != DEC_BF16;
  __shared__ uint32_t lut[kDecLut + kDecSec];
  const DecLds Ls = dec_lds(a.nb, a.stage_words);
  uint32_t* img = reinterpret_cast<uint32_t*>(dsh + Ls.image);
  uint32_t* stage = reinterpret_cast<uint32_t*>(dsh + Ls.stage);
  uint32_t* blk_f = reinterpret_cast<uint32_t*>(dsh + Ls.blk);       // flags per block of the unit
  uint32_t* blk_v = blk_f + 64;                                       // verbatim rank of the block's first
  const int lane = threadIdx.x;
  const int t = blockIdx.y;
  const int bA = blockIdx.x * a.nb;
  const int nbu = min(a.nb, a.kb - bA);
  const int rows = min(16, a.n - 16 * t);
  const uint32_t realmask = rows == 16 ? 0xFFFFu : ((1u << rows) - 1u);
  const uint16_t* flg = a.flags + (size_t)t * a.kb;

  // Chunks and verbatim segments of the tile's blocks before this unit.
  uint32_t ch_before = 0, v_before = 0;
  for (int b0 = 0; b0 < bA; b0 += 64) {
    const int b = b0 + lane;
    uint32_t nch = 0, nv = 0;
    if (b < bA) {
      const uint32_t f = flg[b];
      nch = ((uint32_t)__popc(realmask & ~f) + a.spc - 1) / a.spc;
      nv = __popc(f);
    }
    ch_before += wave_sum(nch);
    v_before += wave_sum(nv);
  }
  // This unit's blocks: flags, chunk counts, exclusive prefixes (lane = block in unit).
  uint32_t f = 0, nch = 0, nv = 0;
  if (lane < nbu) {
    f = flg[bA + lane];
    nch = ((uint32_t)__popc(realmask & ~f) + a.spc - 1) / a.spc;
    nv = __popc(f);
  }
  const uint32_t ch_incl = wave_incl_scan(nch, lane), v_incl = wave_incl_scan(nv, lane);
  const uint32_t unit_chunks = __shfl(ch_incl, 63, 64);
  if (lane < nbu) {
    blk_f[lane] = f;
    blk_v[lane] = a.vprefix[t] + v_before + v_incl - nv;
  }
  const uint32_t c_first = a.cbase[t] + ch_before;
  const uint32_t ch_pre = ch_incl - nch;                       // per block lane

  // Stage the unit's bitstream slice in 1 KB LDS-DMA steps (no VGPRs, no waits until the
  // barrier; words past the stream read as zero), and build the table meanwhile.
  uint32_t wb = 0, nst = 0;
  if (unit_chunks) {
    wb = (a.off[c_first] >> 5) & ~3u;
    const uint32_t we = (a.off[c_first + unit_chunks] >> 5) + 3u;
    nst = min((we - wb + 255u) & ~255u, a.stage_words);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.words, a.words_cap * 4u);
    for (uint32_t i = 0; i < nst; i += 256u)
      lds_dma16(rs, reinterpret_cast<uint8_t*>(stage + i), (wb + i) * 4u + (uint32_t)lane * 16u);
  }
  build_dec_lut(a, lut, reinterpret_cast<uint16_t*>(img), lane);
  __syncthreads();
  // Index and exponent modes: results go straight to the unit's output range (a lane without
  // a finished word stores out of range, which writes nothing).
  constexpr uint32_t kOutBlk = MODE == DEC_IDX ? 512u : 1024u;   // output bytes per block (direct modes)
  const uint32_t rowb = (uint32_t)a.k * 2u;                       // BF16 output row, bytes
  uint8_t* const obase = kDirect ? a.out + ((size_t)t * a.kb + bA) * kOutBlk
                                 : a.out + ((size_t)t * 16 * a.k + (size_t)bA * 64) * 2;
  const __amdgpu_buffer_rsrc_t ors =
      make_rsrc(obase, kDirect ? (uint32_t)nbu * kOutBlk : (uint32_t)(rows - 1) * rowb + (uint32_t)nbu * 128u);

  // Decode: lane -> (block in unit, chunk in block).
  const int bl = lane / a.cpb, j = lane % a.cpb;
  const uint32_t bf = __shfl(f, bl < 64 ? bl : 0, 64);
  const uint32_t bpre = __shfl(ch_pre, bl < 64 ? bl : 0, 64);
  uint32_t cm = realmask & ~bf;                                 // coded rows of the block
  const int ncoded = __popc(cm);
  uint32_t bad = 0;
  if (bl < nbu && j * a.spc < ncoded) {
    const int nrows = min(a.spc, ncoded - j * a.spc);
    int32_t rem4 = nrows * 256;                                 // 4 x symbols left
    const uint32_t c = c_first + bpre + (uint32_t)j;
    const uint32_t p0 = a.off[c] - wb * 32u, p1 = a.off[c + 1] - wb * 32u;
    auto word = [&](uint32_t i) -> uint32_t { return i < nst ? stage[i] : 0u; };
    // Bit window: the 32 bits starting (32 - s) bits into w0 (s = 0: w1 itself).
    const uint32_t b0 = p0 & 31u, wi0 = p0 >> 5;
    uint32_t w0 = b0 ? word(wi0) : 0u, w1 = word(b0 ? wi0 + 1 : wi0);
    const uint32_t* nxp = stage + (b0 ? wi0 + 2 : wi0 + 1);     // next stream word
    const uint32_t* const lastp = stage + (nst ? nst - 1 : 0);
    uint32_t s = b0 ? 32u - b0 : 0u;
    // Output, in decode order: the q-th coded row of block bl holds its 8 index words at
    // bl * 512 + q * 32 (the chunk's rows are consecutive coded rows), so a lane fills its
    // own run of bytes; BF16 mode: at q * rowb + bl * 32 (woff counts q * 32 + word * 4).
    uint32_t woff = (kDirect ? (uint32_t)bl * 512u : 0u) + (uint32_t)(j * a.spc) * 32u;
    const uint32_t lb32 = (uint32_t)bl * 32u;
    uint64_t acc = 0;
    uint32_t a4 = 0;                                            // 4 x indices pending in acc
    // One lookup's worth: append `syms` (n4 / 4 indices), consume L bits, emit a finished word.
    auto step = [&](uint32_t syms, uint32_t n4, uint32_t L, uint32_t v) {
      acc |= (uint64_t)syms << a4;
      a4 += n4;
      rem4 -= (int32_t)n4;
      const int32_t sl = (int32_t)s - (int32_t)L;
      const bool neg = sl < 0;
      w0 = neg ? w1 : w0;
      w1 = neg ? v : w1;
      nxp += (uint32_t)sl >> 31;
      s = (uint32_t)sl & 31u;
      // a4 < 64, so bit 5 is the flush flag; it drives the store offset (out of range when
      // clear), the accumulator shift and the offset step without a branch.
      const uint32_t f32 = a4 & 32u;
      const uint32_t iw = nibbles_to_index_word((uint32_t)acc);
      const uint32_t po = kDirect ? woff : (woff >> 5) * rowb + lb32 + (woff & 31u);
      __builtin_amdgcn_raw_buffer_store_b32(iw, ors, po | ((f32 ^ 32u) << 26), 0, 0);
      acc >>= f32;
      a4 &= 31u;
      woff += f32 >> 3;
    };
    // Long or invalid first code: the secondary entry, or a one-bit placeholder when invalid.
    // (Block 0 of the secondary table is all invalid: it serves invalid primary entries.)
    auto resolve = [&](uint32_t e, uint32_t win) -> uint32_t {
      if (e < (1u << 29)) {
        const uint32_t e2 = lut[kDecLut + (e & 15u) * 8u + ((win >> 19) & 7u)];
        const bool inv = e2 < (1u << 29);
        bad |= inv ? 1u : 0u;
        e = inv ? (1u << 29) | (1u << 20) | (1u << 16) : e2;
      }
      return e;
    };
    while (rem4 >= 16) {
      const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, s);
      uint32_t e = lut[win >> (32 - kDecWin)];
      const uint32_t v = *(nxp < lastp ? nxp : lastp);           // refill candidate
      e = resolve(e, win);
      step(e & 0xFFFFu, e >> 27, (e >> 16) & 15u, v);
    }
    while (rem4 > 0) {
      const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, s);
      uint32_t e = lut[win >> (32 - kDecWin)];
      const uint32_t v = *(nxp < lastp ? nxp : lastp);
      e = resolve(e, win);
      step(e & 15u, 4u, (e >> 20) & 15u, v);
    }
    const uint32_t pos = (uint32_t)(nxp - stage) * 32u - 32u - s;   // bits consumed from the slice start
    if (pos != p1) bad = 1;
  }
  if (bad) atomicOr(a.err, 1u);

  // Write the unit's output in its final layout.  Row r of block b is coded unless flagged
  // verbatim; a coded row's words sit at its rank among the block's coded rows.  The words
  // went out in decode order (this workgroup's stores are complete at the barrier); they come
  // back through the (now free) table scratch and stage in 1 KB LDS-DMA steps, bypassing the
  // vector cache, and every line of the unit's output is written once.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  uint8_t* const back = reinterpret_cast<uint8_t*>(img);
  if constexpr (kDirect) {
    for (uint32_t i = 0; i < (uint32_t)nbu * 512u; i += 1024u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_ptr_t)(back + i), 16, i + (uint32_t)lane * 16u, 0, 0, 1);
  } else {
    // Row q's run of nbu * 32 bytes lands at back + q * run: a 1 KB step covers several rows.
    const uint32_t run = (uint32_t)nbu * 32u, total = (uint32_t)rows * run;
    for (uint32_t i = 0; i < total; i += 1024u) {
      const uint32_t o = i + (uint32_t)lane * 16u, q = o / run;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_ptr_t)(back + i), 16, o < total ? q * rowb + (o - q * run) : kOob,
                                               0, 0, 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  if constexpr (MODE == DEC_IDX) {
    // 16-byte piece p: block p / 32, sub-tile (p / 8) % 4, rows 2 (p % 8) and 2 (p % 8) + 1.
    u32x4* dst = reinterpret_cast<u32x4*>(obase);
    for (int p = lane; p < nbu * 32; p += 64) {
      const int b = p >> 5, g = (p >> 3) & 3, r = (p & 7) * 2;
      const uint32_t coded = realmask & ~blk_f[b];
      const uint32_t q = __popc(coded & ((1u << r) - 1u));
      const u32x2* src = reinterpret_cast<const u32x2*>(back + b * 512 + g * 8);
      const u32x2 z{0, 0};
      const u32x2 w0 = ((coded >> r) & 1u) ? src[q * 4] : z;
      const u32x2 w1 = ((coded >> (r + 1)) & 1u) ? src[(q + ((coded >> r) & 1u)) * 4] : z;
      dst[p] = u32x4{w0.x, w0.y, w1.x, w1.y};
    }
  } else if constexpr (MODE == DEC_EXP) {
    // 16-byte piece p: block p / 64, sub-tile (p / 16) % 4, row p % 16.  Verbatim rows take
    // their raw exponents, padding rows zeros.
    u32x4* dst = reinterpret_cast<u32x4*>(obase);
    for (int p = lane; p < nbu * 64; p += 64) {
      const int b = p >> 6, g = (p >> 4) & 3, r = p & 15;
      const uint32_t fb = blk_f[b];
      u32x4 o{0, 0, 0, 0};
      if ((fb >> r) & 1u) {
        const uint32_t v = blk_v[b] + __popc(fb & ((1u << r) - 1u));
        o = *reinterpret_cast<const u32x4*>(a.vexp + (size_t)v * 64 + g * 16);
      } else if (r < rows) {
        const uint32_t q = (uint32_t)r - __popc(fb & ((1u << r) - 1u));
        const u32x2 iw = *reinterpret_cast<const u32x2*>(back + b * 512 + q * 32 + g * 8);
        const u32x2 e0 = index_word_to_exps(iw.x, a.tab), e1 = index_word_to_exps(iw.y, a.tab);
        o = u32x4{e0.x, e0.y, e1.x, e1.y};
      }
      dst[p] = o;
    }
  } else {
    // BF16 rows: 16-byte piece p = 8 weights; row p / (nbu*8), then block, sub-tile, half.
    // Four pieces a lane at a time: their loads all go out before the first store.
    const uint32_t rs = (uint32_t)nbu * 32u;
    const int per_row = nbu * 8, total = rows * per_row;
    constexpr int kPieces = 4;
    for (int p0 = lane; p0 < total; p0 += 64 * kPieces) {
      u32x2 sv[kPieces], e[kPieces];
      size_t dsto[kPieces];
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const int p = min(p0 + 64 * u, total - 1);
        const int r = p / per_row, q = p - r * per_row;
        const int b = q >> 3, g = (q >> 1) & 3, h = q & 1;
        const uint32_t fb = blk_f[b];
        const uint32_t vb = __popc(fb & ((1u << r) - 1u));
        if ((fb >> r) & 1u) {
          e[u] = *reinterpret_cast<const u32x2*>(a.vexp + (size_t)(blk_v[b] + vb) * 64 + g * 16 + h * 8);
        } else {
          e[u] = index_word_to_exps(*reinterpret_cast<const uint32_t*>(back + ((uint32_t)r - vb) * rs + b * 32 + (g * 2 + h) * 4),
                                    a.tab);
        }
        const size_t sub = ((size_t)t * a.kb * 4 + (size_t)(bA + b) * 4 + g) * 16 + r;
        sv[u] = *reinterpret_cast<const u32x2*>(a.sm + sub * 16 + h * 8);
        dsto[u] = ((size_t)r * a.k + (size_t)b * 64 + g * 16 + h * 8) * 2;
      }
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        if (p0 + 64 * u >= total) break;
        u32x4 o;
        o.x = bf16_pairs_from(sv[u].x, e[u].x, 0);
        o.y = bf16_pairs_from(sv[u].x, e[u].x, 1);
        o.z = bf16_pairs_from(sv[u].y, e[u].y, 0);
        o.w = bf16_pairs_from(sv[u].y, e[u].y, 1);
        *reinterpret_cast<u32x4*>(obase + dsto[u]) = o;
      }
    }
  }
}

// =========================================================================================
// Register-image decoder (chunks of at most 8 coded rows: chunk <= 512 symbols).
//
// One wave per unit (tile t, nb whole blocks), lane = (block in unit, chunk slot in block) as
// above; W waves a workgroup share one 2^12-entry table of up to five symbols an entry (16 KB
// of LDS, built once per workgroup).  Each lane keeps its chunk's decoded rows in VGPRs (64
// words: eight rows of eight words of 4-bit indices in decode order), so LDS holds only the
// bitstream slices and every unit of a large matrix is resident at once; the wave writes its
// output lines once, whole, when the unit is done (HBM traffic: the bitstream in, the output
// out).  A VGPR cannot be indexed per lane, so words reach the image through a small LDS
// buffer per lane, in phases of two rows: phase h ends when every lane of the wave has
// decoded its rows 2h, 2h + 1, and its 16 words are then copied to statically indexed VGPRs.
// A lookup may run up to four symbols past a phase (less than a word), which land in the
// buffer's 17th word and carry over.
//   Table entry: total code length of the entry's symbols in bits 0-3, 4 x symbol count in
//   bits 4-8, the symbols in bits 12-31 (first in bits 12-15).  Length and count 0: the window
//   starts a 13-bit code (bits 9-11: block of two secondary entries chosen by the 13th bit;
//   block 0 is all invalid) or no code; such an entry changes nothing, and the lane leaves the
//   hot loop for one slow step, which also takes the last one to four symbols of a chunk one
//   at a time (a lookup must not take symbols of the next chunk).  The encoders limit codes to
//   12 bits, so their blobs never take that path for a code; a blob written at the format's
//   13-bit limit does, and each such code costs its wave dearly: the lane waits in place until
//   every other lane has finished the phase, then decodes the rest of it alone (on gate_proj
//   written at 13 bits, where a wave meets one in most phases: transcode 40.7 against 33.4 us).
// =========================================================================================
constexpr int kRowWin = 12;                 // lookup window, bits
constexpr int kRowLut = 1 << kRowWin;       // primary entries
constexpr int kRowSecBlocks = 8;            // secondary blocks of 2 (block 0: invalid)
constexpr int kRowSec = 2 * kRowSecBlocks;
constexpr int kRowMaxSyms = 5;              // symbols an entry
constexpr int kPhaseRows = 2;               // rows a phase
constexpr int kPhaseWords = 8 * kPhaseRows; // words a phase
constexpr int kPhases = 8 / kPhaseRows;     // phases of the longest chunk (eight rows)
constexpr int kBufStride = kPhaseWords + 1; // words of one lane's phase buffer (odd: spreads LDS banks)
constexpr uint32_t kBufBytes = 64u * kBufStride * 4u;    // one wave's phase buffers
constexpr uint32_t kRowTmpBytes = kRowLut * 2u;          // table-build scratch (u16 a window)

struct RowDecArgs {
  const uint32_t* words;
  const uint32_t* off;
  const uint32_t* cbase;
  const uint16_t* flags;
  const uint32_t* vprefix;
  const uint8_t* vexp;
  const uint8_t* sm;
  uint8_t* out;
  uint32_t* err;
  uint32_t words_cap;
  int32_t n, k, kb;
  int32_t spc, cpb, nb;     // coded segments per chunk (<= 8), chunk slots per block, blocks per unit
  uint32_t spc_magic;       // ceil(2^16 / spc): q / spc = (q * spc_magic) >> 16 for q < 16
  int32_t units_per_tile, units;
  uint32_t stage_words;     // LDS words for one unit's bitstream slice (host bound, multiple of 256)
  uint32_t stage_off;       // byte offset of the stages in the dynamic LDS block
  uint32_t tab[4];          // palette, 16 bytes
  uint32_t len_lo, len_hi;  // code lengths of symbols 0-7 and 8-15, a nibble each
  uint8_t len[16];
  uint16_t code[16];
  uint32_t pbase;           // first 12-bit prefix of a 13-bit code
  uint32_t nblk;            // prefixes of 13-bit codes (consecutive from pbase), <= 7
  uint32_t sec[kRowSec];    // secondary entries (same format as the primary ones)
  const uint32_t* lut_src;  // the primary table, built on the host at bind time, or null (built here)
};

// Dynamic LDS of one workgroup of W waves: [phase buffers (before the decode: the table-build
// scratch)][W stages].
__host__ __device__ inline uint32_t row_buf_area(int W) {
  return std::max<uint32_t>(kRowTmpBytes, (uint32_t)W * kBufBytes);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS accesses, not for its global
// loads, so the stage DMAs stay in flight across it (__syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(63) & ~0x0F00);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ void build_row_lut(const RowDecArgs& a, uint32_t* lut, uint16_t* tmp) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < kRowLut / 2; i += nt) reinterpret_cast<uint32_t*>(tmp)[i] = 0;
  lds_barrier();
  for (int s = 0; s < 16; ++s) {
    const int L = a.len[s];
    if (L == 0 || L > kRowWin) continue;
    const uint32_t lo = (uint32_t)a.code[s] << (kRowWin - L), cnt = 1u << (kRowWin - L);
    for (uint32_t i = tid; i < cnt; i += nt) tmp[lo + i] = (uint16_t)(s | (L << 4) | 0x100);
  }
  lds_barrier();
  // Four windows a thread at a time (independent chains of table reads).
  constexpr int kIlp = 4;
  for (int w0 = tid; w0 < kRowLut; w0 += nt * kIlp) {
    uint32_t used[kIlp], n[kIlp], syms[kIlp], first[kIlp];
#pragma unroll
    for (int q = 0; q < kIlp; ++q) {
      const int w = min(w0 + q * nt, kRowLut - 1);
      first[q] = tmp[w];
      used[q] = (first[q] >> 4) & 15u;
      n[q] = 1;
      syms[q] = first[q] & 15u;
    }
#pragma unroll
    for (int j = 1; j < kRowMaxSyms; ++j) {
#pragma unroll
      for (int q = 0; q < kIlp; ++q) {
        const int w = min(w0 + q * nt, kRowLut - 1);
        const uint32_t ej = tmp[(w << used[q]) & (kRowLut - 1)];
        const uint32_t lj = (ej >> 4) & 15u;
        const bool ok = (n[q] == (uint32_t)j) && (ej & 0x100u) && used[q] + lj <= (uint32_t)kRowWin;
        syms[q] |= ok ? (ej & 15u) << (4 * j) : 0u;
        used[q] += ok ? lj : 0u;
        n[q] += ok ? 1u : 0u;
      }
    }
#pragma unroll
    for (int q = 0; q < kIlp; ++q) {
      const int w = w0 + q * nt;
      if (w >= kRowLut) continue;
      uint32_t entry;
      if (first[q] & 0x100u) {
        entry = (syms[q] << 12) | (4u * n[q] << 4) | used[q];
      } else {
        const uint32_t i = (uint32_t)w - a.pbase;   // a 13-bit code's prefix: secondary block i + 1
        entry = i < a.nblk ? (i + 1u) << 9 : 0u;
      }
      lut[w] = entry;
    }
  }
  // Constant indices: the entries come from the kernel arguments through scalar loads (an
  // indexed read would be a vector load, and waiting for it would wait for the stage DMAs).
#pragma unroll
  for (int i = 0; i < kRowSec; ++i)
    if (tid == i) lut[kRowLut + i] = a.sec[i];
  lds_barrier();
}

// Smallest value v (< 2^BITS) over the lanes where act is set, 2^BITS when there are none; the
// result is wave-uniform.  Bit slices from the top: the candidates keep the lanes whose bits
// so far equal the minimum's (ballots only, no LDS round trips).
template <int BITS>
__device__ __forceinline__ uint32_t wave_min_small(uint32_t v, bool act) {
  uint64_t cand = __builtin_amdgcn_ballot_w64(act);
  if (!cand) return 1u << BITS;
  uint32_t r = 0;
#pragma unroll
  for (int p = BITS - 1; p >= 0; --p) {
    const uint64_t z = cand & __builtin_amdgcn_ballot_w64(((v >> p) & 1u) == 0u);
    if (z) cand = z;
    else r |= 1u << p;
  }
  return r;
}

// Sequential nibbles n0..n7 (n_i at bits 4i) -> 8 exponent bytes in column order.
__device__ __forceinline__ u32x2 seq_word_to_exps(uint32_t v, const uint32_t tab[4]) {
  const uint32_t ev = lookup16(v & 0x0F0F0F0Fu, tab);          // E0 E2 E4 E6
  const uint32_t od = lookup16((v >> 4) & 0x0F0F0F0Fu, tab);   // E1 E3 E5 E7
  return u32x2{perm(od, ev, 0x05010400u), perm(od, ev, 0x07030602u)};
}

// 4 x symbol count of a table entry, and a slice pointer moved on by 0 or 1 words, each as the
// single ALU instruction it is (the compiler otherwise splits them into shift-and-mask pairs
// in the decode loop, which is bound by instruction issue).
__device__ __forceinline__ uint32_t entry_n4(uint32_t e) {
  uint32_t r;
  asm("v_bfe_u32 %0, %1, 4, 5" : "=v"(r) : "v"(e));
  return r;
}
typedef const __attribute__((address_space(3))) uint32_t* lds_cu32p;
__device__ __forceinline__ lds_cu32p advance_word(lds_cu32p p, uint32_t step) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(r) : "v"(step), "v"((uint32_t)(uintptr_t)p));
  return (lds_cu32p)(uintptr_t)r;
}

// One unit (wave `wave` of the workgroup, unit u).  first: the workgroup's first unit, whose
// stage DMA overlaps the table build (every wave of the workgroup takes part in the build, unit
// or not); later units wait for their own stage only.
template <int MODE>
__device__ __forceinline__ void decode_unit(const RowDecArgs& a, uint32_t* lut, uint8_t* dsh, int u, int wave,
                                            bool first) {
  const int lane = threadIdx.x & 63;
  const bool unit_ok = u < a.units;
  const int t = unit_ok ? u / a.units_per_tile : 0;
  const int bA = unit_ok ? (u - t * a.units_per_tile) * a.nb : 0;
  const int nbu = unit_ok ? min(a.nb, a.kb - bA) : 0;
  const int rows = min(16, a.n - 16 * t);
  const uint32_t realmask = rows >= 16 ? 0xFFFFu : ((1u << rows) - 1u);
  const uint16_t* flg = a.flags + (size_t)t * a.kb;
  uint32_t* stage = reinterpret_cast<uint32_t*>(dsh + a.stage_off + (uint32_t)wave * a.stage_words * 4u);
  uint32_t* const buf = reinterpret_cast<uint32_t*>(dsh + (uint32_t)wave * kBufBytes) + lane * kBufStride;
  // A table built at bind time: its 16 one-kilobyte pieces go to LDS by LDS-DMA before any
  // other load (wave w takes pieces w, w + W, ...), so they arrive with the first round trips.
  if (first && a.lut_src) {
    const int W = (int)(blockDim.x >> 6);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lut_src, kRowLut * 4u);
    for (int pc = wave; pc < kRowLut * 4 / 1024; pc += W)
      lds_dma16(rl, reinterpret_cast<uint8_t*>(lut) + pc * 1024, (uint32_t)pc * 1024u + (uint32_t)lane * 16u);
  }

  // Chunks and verbatim segments of the tile's blocks before this unit; then this unit's
  // blocks (lane = block in unit): flags, chunk counts and exclusive prefixes.
  uint32_t ch_before = 0, v_before = 0;
  for (int c0 = 0; c0 < bA; c0 += 64) {
    const int b = c0 + lane;
    uint32_t nch = 0, nv = 0;
    if (b < bA) {
      const uint32_t f = flg[b];
      nch = ((uint32_t)__popc(realmask & ~f) + a.spc - 1) / a.spc;
      nv = __popc(f);
    }
    ch_before += wave_sum(nch);
    v_before += wave_sum(nv);
  }
  uint32_t f = 0, nch = 0, nv = 0;
  if (lane < nbu) {
    f = flg[bA + lane];
    nch = ((uint32_t)__popc(realmask & ~f) + a.spc - 1) / a.spc;
    nv = __popc(f);
  }
  const uint32_t ch_incl = wave_incl_scan(nch, lane), v_incl = wave_incl_scan(nv, lane);
  const uint32_t unit_chunks = __shfl(ch_incl, 63, 64);
  const uint32_t c_first = unit_ok ? a.cbase[t] + ch_before : 0u;
  const uint32_t vblk = unit_ok ? a.vprefix[t] + v_before + v_incl - nv : 0u;   // per block lane

  // Lane -> (block in unit, chunk slot in block) and this lane's chunk.
  const int bl = lane / a.cpb, j = lane - (lane / a.cpb) * a.cpb;
  const int src = bl < 64 ? bl : 0;
  const uint32_t bf = __shfl(f, src, 64);
  const uint32_t bpre = __shfl(ch_incl - nch, src, 64);
  const uint32_t bvr = __shfl(vblk, src, 64);
  const uint32_t cm = realmask & ~bf;                           // coded rows of the block
  const int ncoded = __popc(cm);
  const bool lane_ok = bl < nbu;
  const bool has_chunk = lane_ok && j * a.spc < ncoded;
  const int nrows = has_chunk ? min(a.spc, ncoded - j * a.spc) : 0;
  const uint32_t c = c_first + bpre + (uint32_t)j;
  int wmax_rows = nrows;                                        // most rows of any chunk of the wave
  for (int o = 32; o > 0; o >>= 1) wmax_rows = max(wmax_rows, __shfl_xor(wmax_rows, o, 64));
  wmax_rows = __builtin_amdgcn_readfirstlane(wmax_rows);

  // Every bit offset the unit needs (slice ends, the lane's chunk) in one round trip, then the
  // slice staged (1 KB LDS-DMA steps; words past the stream read zero).  Nothing below waits
  // on a global load until the decode itself: loads retire in order, so such a wait would also
  // wait for every DMA issued before it.
  uint32_t o_first = 0, o_end = 0, o_c0 = 0, o_c1 = 0;
  if (unit_chunks) {
    o_first = a.off[c_first];
    o_end = a.off[c_first + unit_chunks];
  }
  if (has_chunk) {
    o_c0 = a.off[c];
    o_c1 = a.off[c + 1];
  }
  uint32_t wb = 0, nst = 0;
  if (unit_chunks) {
    wb = (o_first >> 5) & ~3u;
    const uint32_t we = (o_end >> 5) + 3u;
    nst = min((we - wb + 255u) & ~255u, a.stage_words);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.words, a.words_cap * 4u);
    for (uint32_t i = 0; i < nst; i += 256u)
      lds_dma16(rs, reinterpret_cast<uint8_t*>(stage + i), (wb + i) * 4u + (uint32_t)lane * 16u);
  }
  const uint32_t p0 = has_chunk ? o_c0 - wb * 32u : 0u, p1 = has_chunk ? o_c1 - wb * 32u : 0u;

  if (first) {
    if (a.lut_src) {
      // The secondary entries from the kernel arguments; then every wave's table pieces (and
      // stage) landed before any wave reads the table.
      const int tid = (int)threadIdx.x;
#pragma unroll
      for (int i = 0; i < kRowSec; ++i)
        if (tid == i) lut[kRowLut + i] = a.sec[i];
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
    } else {
      build_row_lut(a, lut, reinterpret_cast<uint16_t*>(dsh));   // LDS barriers only: the DMAs stay in flight
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                    // this wave's stage (and earlier stores)
  if (!unit_ok) return;

  // Bit window: the 32 bits starting (32 - s) bits into w0 (s = 0: w1 itself); np: the next
  // word of the slice.
  const uint32_t b0 = p0 & 31u, wi0 = p0 >> 5;
  uint32_t w0 = b0 ? stage[wi0] : 0u, w1 = stage[b0 ? wi0 + 1 : wi0];
  lds_cu32p np = (lds_cu32p)(stage + (b0 ? wi0 + 2 : wi0 + 1));
  uint32_t s = b0 ? 32u - b0 : 0u;
  int32_t rem4 = nrows * 256;                                   // 4 x symbols left
  uint32_t lo = 0;                                              // the word in progress (4-bit indices)
  uint32_t a4 = 0;                                              // its bits filled
  uint32_t* wp = buf;                                           // its place in the phase buffer
  uint32_t bad = 0;
  // Index and exponent output: every two phases (four rows) are written as soon as they are
  // decoded, so the output writes overlap the decode of later phases and only two phases' words
  // are held in VGPRs.  A lane's four rows of one sub-tile are contiguous: 64 bytes of exponents
  // (a whole 64-byte segment: 1.01x the output bytes in HBM writes) or 32 bytes of indices (half
  // a segment, the other half two phases later: 1.47x).  Written a phase at a time (16 or 32
  // bytes) the output took 2.8x its bytes; written at the end of the chunk from an eight-row
  // register image, 1.0x but slower (gate transcode 53.6 against 49.5 us, exponents 54.4 against
  // 51.0 at 512-symbol chunks).  BF16 output: a row is 128 contiguous bytes of W, whole lines, so
  // it is written a phase (two rows) at a time, with the rows' sign+mantissa bytes loaded a phase
  // ahead.
  constexpr bool kBf16 = MODE == DEC_BF16;
  uint32_t grp[kBf16 ? 1 : kPhaseWords];         // the even phase's words, written with the odd one's
  int hdone = 0;

  // Output places: chunk row q is the (j spc + q)-th coded row of the block; its 16-weight
  // groups g go to sub-tile (t, 4 blk + g) of the output stream.
  uint32_t first_rows = cm;
  for (int i = 0; i < j * a.spc && first_rows; ++i) first_rows &= first_rows - 1u;
  uint32_t rowq[8];
  {
    uint32_t mm = first_rows;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      rowq[q] = __builtin_ctz(mm | 0x10000u);
      mm &= mm - 1u;
    }
  }
  const uint32_t rowb = (uint32_t)a.k * 2u;                   // a BF16 output row, bytes
  const __amdgpu_buffer_rsrc_t ors =
      MODE == DEC_IDX ? make_rsrc(a.out + (size_t)t * a.k * 8 + (size_t)bA * 512, (uint32_t)nbu * 512u)
      : MODE == DEC_EXP ? make_rsrc(a.out + (size_t)t * a.k * 16 + (size_t)bA * 1024, (uint32_t)nbu * 1024u)
                        : make_rsrc(a.out + (size_t)t * 16 * rowb, (uint32_t)(rows - 1) * rowb + rowb);
  // BF16: the tile's sign+mantissa sub-tiles; row r's 16 bytes of sub-tile (t, 4 blk + g).
  const uint32_t blk = (uint32_t)(bA + bl);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.sm + (size_t)t * a.k * 16, (uint32_t)a.k * 16u);
  auto load_sm = [&](uint32_t row, bool ok, u32x4 sv[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sv[g] = bload16(srs, ok ? ((blk * 4 + g) * 16 + row) * 16 : kOob);
  };
  // 16-byte piece p (weights 8p .. 8p + 7) of BF16 row `row`: sign+mantissa from sv, exponents e.
  auto put_bf16 = [&](uint32_t row, bool ok, const u32x4 sv[4], int p, u32x2 e) {
    const uint32_t s0 = (p & 1) ? sv[p >> 1].z : sv[p >> 1].x, s1 = (p & 1) ? sv[p >> 1].w : sv[p >> 1].y;
    const u32x4 o{bf16_pairs_from(s0, e.x, 0), bf16_pairs_from(s0, e.x, 1), bf16_pairs_from(s1, e.y, 0),
                  bf16_pairs_from(s1, e.y, 1)};
    __builtin_amdgcn_raw_buffer_store_b128(o, ors, ok ? row * rowb + blk * 128u + (uint32_t)p * 16u : kOob, 0, 0);
  };
  u32x4 svp[kBf16 ? kPhaseRows : 1][4];         // the current phase's rows' sign+mantissa bytes
  // Rows q0 .. q0 + nq - 1 (words w[8 i .. 8 i + 7] of 4-bit indices in sequence order for row
  // q0 + i) to the index or exponent output, sub-tile by sub-tile.
  // Index rows go out in pairs: two adjacent rows of a sub-tile are 16 contiguous bytes, one
  // store instead of two (the scattered output stores, not the decode, had become the larger
  // cost: half the store instructions and twice the bytes a lane-request).  A pair split by a
  // verbatim or padding row takes two 8-byte stores, in a branch the wave skips when no lane
  // needs it.
  auto put_rows = [&](int q0, int nq, const uint32_t* w) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int i = 0; i < nq; i += (MODE == DEC_IDX ? 2 : 1)) {
        const int q = q0 + i;
        const uint32_t sub = (uint32_t)(bl * 4 + g) * 16 + rowq[q];
        if constexpr (MODE == DEC_IDX) {
          const u32x2 v{nibbles_to_index_word(w[8 * i + 2 * g]), nibbles_to_index_word(w[8 * i + 2 * g + 1])};
          if (i + 1 < nq) {
            const u32x2 v1{nibbles_to_index_word(w[8 * (i + 1) + 2 * g]), nibbles_to_index_word(w[8 * (i + 1) + 2 * g + 1])};
            const bool pair = q + 1 < nrows && rowq[q + 1] == rowq[q] + 1u;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v1.x, v1.y}, ors, pair ? sub * 8 : kOob, 0, 0);
            if (!pair && q < nrows) {
              __builtin_amdgcn_raw_buffer_store_b64(v, ors, sub * 8, 0, 0);
              const uint32_t sub1 = (uint32_t)(bl * 4 + g) * 16 + rowq[q + 1];
              __builtin_amdgcn_raw_buffer_store_b64(v1, ors, q + 1 < nrows ? sub1 * 8 : kOob, 0, 0);
            }
          } else {
            __builtin_amdgcn_raw_buffer_store_b64(v, ors, q < nrows ? sub * 8 : kOob, 0, 0);
          }
        } else {
          const u32x2 e0 = seq_word_to_exps(w[8 * i + 2 * g], a.tab), e1 = seq_word_to_exps(w[8 * i + 2 * g + 1], a.tab);
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{e0.x, e0.y, e1.x, e1.y}, ors, q < nrows ? sub * 16 : kOob, 0, 0);
        }
      }
    }
  };

  // One lookup's state change: e = (length, 4 x count, symbols) as in the table.  The word in
  // progress is stored at every lookup (complete or not), so a finished word is already in the
  // buffer when wp moves on; the symbols past it start the next word (a word boundary is never
  // crossed at a4 = 0: an entry holds at most 20 bits, so the shift by 32 - a4 is then unused).
  // The two halves are separate so that a loop can move the window and send the next lookup's
  // table read before it places this entry's symbols: the wave issues in order, so symbols
  // placed first would sit on the serial chain from one table read to the next.
  auto step = [&](uint32_t e, uint32_t v) {                    // the bit window
    const int32_t sl = (int32_t)s - (int32_t)(e & 15u);
    const bool neg = sl < 0;
    s = (uint32_t)sl & 31u;
    w0 = neg ? w1 : w0;
    w1 = neg ? v : w1;
    np = advance_word(np, (uint32_t)sl >> 31);
  };
  // The symbols: put stores the word in progress with them (first in a pipelined lookup, so the
  // store is not the LDS operation the next lookup's wait ends on), place moves on.
  auto put = [&](uint32_t e) { *wp = ((e >> 12) << a4) | lo; };
  auto place = [&](uint32_t e) {
    const uint32_t n4 = entry_n4(e), sy = e >> 12;
    const uint32_t lo2 = (sy << a4) | lo;
    const uint32_t a4n = a4 + n4;
    const uint32_t carry = sy >> ((32u - a4) & 31u);
    const bool done = a4n >= 32u;
    lo = done ? carry : lo2;
    a4 = a4n & 31u;
    wp += done ? 1 : 0;
    rem4 -= (int32_t)n4;
  };
  auto apply = [&](uint32_t e, uint32_t v) {
    put(e);
    step(e, v);
    place(e);
  };
  // The compiler would otherwise fold a loop's two reads of the next entry (before the loop and
  // at its end) into one read at the top of the loop, which undoes the pipelining: a barrier to
  // memory motion (no instruction) after the end-of-loop read prevents it.
  auto keep_reads_here = []() { asm volatile("" ::: "memory"); };
  auto lookup = [&]() { return lut[__builtin_amdgcn_alignbit(w0, w1, s) >> (32 - kRowWin)]; };

  if constexpr (kBf16) {
#pragma unroll
    for (int qq = 0; qq < kPhaseRows; ++qq) load_sm(rowq[qq], qq < nrows, svp[qq]);
  }
#pragma unroll
  for (int h = 0; h < kPhases; ++h) {
    if (kPhaseRows * h >= wmax_rows) break;
    // Phase h needs symbols up to 128 (h + 1) of the chunk: rem4 down to lim.  Whole table
    // entries are taken while rem4 is above fast_lim: in a phase that ends inside the chunk a
    // lookup may run up to four symbols into the next phase (they start the next word), so
    // fast_lim keeps five symbols' room; in the chunk's last phase entries run to the chunk's
    // end, and the symbols a lookup takes past it stay in the word in progress, which is never
    // written out (the chunk ends on a word boundary); the end check below takes their bits off.
    const int32_t lim = max(4 * (64 * nrows - 64 * kPhaseRows * (h + 1)), 0);
    const int32_t fast_lim = lim > 0 ? max(lim, 4 * kRowMaxSyms - 1) : 0;
    while (true) {
      // A run of lookups that every lane still in the hot loop needs: a lookup takes at most
      // five symbols, so a lane with rem4 above fast_lim takes at least ceil((rem4 - fast_lim)
      // / 20) more.  The run has a wave-uniform trip count and no per-lookup exit test, which
      // costs about 40 % of a lookup's time (a compare, mask updates and a branch that waits
      // for them).  An entry of count 0 (a 13-bit code) changes no state, so a lane that meets
      // one waits in place until the checked loop below.
      {
        const bool act = rem4 > fast_lim;
        const uint32_t want = act ? min((uint32_t)(rem4 - fast_lim + 4 * kRowMaxSyms - 1) / (4u * kRowMaxSyms), 31u) : 0u;
        const uint32_t run = wave_min_small<5>(want, act);
        if (run < 32u && act) {
          // LDS reads still in flight here would otherwise make the compiler wait for them at
          // the top of every lookup (the wait sits at the loop header, where the paths merge).
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(63) & ~0x0F00);
          // Pipelined by one lookup: the reads after the last one are not used (LDS reads past
          // the stage stay inside the workgroup's LDS or read zeros).
          uint32_t e = lookup(), v = *np;
          for (uint32_t i = 0; i < run; ++i) {
            put(e);
            step(e, v);
            const uint32_t en = lookup(), vn = *np;
            keep_reads_here();
            place(e);
            e = en;
            v = vn;
          }
        }
      }
      // Hot loop: whole table entries, each lane until its own limit (pipelined the same way).
      if (rem4 > fast_lim) {
        uint32_t e = lookup(), v = *np;                         // entry, refill candidate
        while (true) {
          put(e);
          step(e, v);
          const uint32_t en = lookup(), vn = *np;
          keep_reads_here();
          place(e);
          if (entry_n4(e) == 0u || rem4 <= fast_lim) break;     // a 13-bit code or no code; or done
          e = en;
          v = vn;
        }
      }
      const bool need = rem4 > lim;
      if (!__builtin_amdgcn_ballot_w64(need)) break;
      if (need) {                                               // one symbol the slow way
        const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, s);
        uint32_t e = lut[win >> (32 - kRowWin)];
        const uint32_t v = *np;
        if (((e >> 4) & 31u) == 0u) {
          const uint32_t e2 = lut[kRowLut + ((e >> 9) & 7u) * 2u + ((win >> (31 - kRowWin)) & 1u)];
          const bool inv = ((e2 >> 4) & 31u) == 0u;
          bad |= inv ? 1u : 0u;
          e = inv ? (4u << 4) | 1u : e2;                        // invalid: one bit, symbol 0
        } else {
          const uint32_t sym = (e >> 12) & 15u;
          const uint32_t L = ((sym < 8 ? a.len_lo : a.len_hi) >> ((sym & 7u) * 4u)) & 15u;
          e = (sym << 12) | (4u << 4) | (L ? L : 1u);
        }
        apply(e, v);
      }
    }
    // Phase done for every lane: its rows 2h, 2h + 1 (16 finished words) to the output or the
    // image; the word in progress (a lookup's symbols past the phase) stays in lo and becomes
    // the buffer's first word.
    if constexpr (!kBf16) {
      if (h & 1) {
        uint32_t w[2 * kPhaseWords];
#pragma unroll
        for (int i = 0; i < kPhaseWords; ++i) {
          w[i] = grp[i];
          w[kPhaseWords + i] = buf[i];
        }
        put_rows(kPhaseRows * (h - 1), 2 * kPhaseRows, w);
      } else {
#pragma unroll
        for (int i = 0; i < kPhaseWords; ++i) grp[i] = buf[i];
      }
      hdone = h + 1;
    } else {
      uint32_t w[kPhaseWords];
#pragma unroll
      for (int i = 0; i < kPhaseWords; ++i) w[i] = buf[i];
#pragma unroll
      for (int qq = 0; qq < kPhaseRows; ++qq) {
        const int q = kPhaseRows * h + qq;
#pragma unroll
        for (int pc = 0; pc < 8; ++pc) put_bf16(rowq[q], q < nrows, svp[qq], pc, seq_word_to_exps(w[8 * qq + pc], a.tab));
      }
      if (h + 1 < kPhases) {   // the next phase's rows, loaded while it is decoded
#pragma unroll
        for (int qq = 0; qq < kPhaseRows; ++qq) {
          const int q = kPhaseRows * (h + 1) + qq;
          load_sm(rowq[q], q < nrows, svp[qq]);
        }
      }
    }
    wp = buf;
  }
  if (has_chunk) {
    // Bits consumed from the slice start, less the codes of the symbols taken past the chunk's
    // end (-rem4 / 4 of them, in the low nibbles of the word in progress).
    uint32_t over = 0;
#pragma unroll
    for (int i = 0; i < kRowMaxSyms - 1; ++i) {
      const uint32_t sym = (lo >> (4 * i)) & 15u;
      const uint32_t L = ((sym < 8 ? a.len_lo : a.len_hi) >> ((sym & 7u) * 4u)) & 15u;
      over += 4 * i < -rem4 ? L : 0u;
    }
    const uint32_t pos = (uint32_t)(np - (lds_cu32p)stage) * 32u - 32u - s - over;
    if (pos != p1) bad = 1;
  }
  if (bad) atomicOr(a.err, 1u);

  if constexpr (!kBf16) {
    // A last, unpaired phase (constant row numbers: rowq is indexed at compile time).
    static_for<0, kPhases / 2>([&](auto pc) {
      constexpr int hp = 2 * decltype(pc)::value;
      if (hdone == hp + 1) put_rows(kPhaseRows * hp, kPhaseRows, grp);
    });
  }
  // The lane's share of the block's other rows (rows j spc .. (j + 1) spc - 1 that are verbatim
  // or padding): the verbatim exponents or zeros.
  uint32_t other = lane_ok ? ~cm & (((1u << a.spc) - 1u) << (j * a.spc)) & 0xFFFFu : 0u;
  if constexpr (MODE == DEC_IDX) {
    // Index stream: row r of sub-tile (t, 4 blk + g) at ((t k/16 + 4 blk + g) 16 + r) 8.
    while (other) {
      const uint32_t r = __builtin_ctz(other);
      other &= other - 1u;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0, 0}, ors, ((uint32_t)(bl * 4 + g) * 16 + r) * 8, 0, 0);
    }
  } else if constexpr (MODE == DEC_EXP) {
    // Exponent bytes in the sign+mantissa sub-tile layout.
    while (other) {
      const uint32_t r = __builtin_ctz(other);
      other &= other - 1u;
      const bool verb = (bf >> r) & 1u;
      const uint8_t* ve = a.vexp + (size_t)(bvr + __popc(bf & ((1u << r) - 1u))) * 64;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 o = verb ? *reinterpret_cast<const u32x4*>(ve + g * 16) : u32x4{0, 0, 0, 0};
        __builtin_amdgcn_raw_buffer_store_b128(o, ors, ((uint32_t)(bl * 4 + g) * 16 + r) * 16, 0, 0);
      }
    }
  } else {
    // BF16 rows: verbatim rows from their raw exponents; padding rows are not part of W.
    while (other) {
      const uint32_t r = __builtin_ctz(other);
      other &= other - 1u;
      if (r >= (uint32_t)rows) continue;
      const uint8_t* ve = a.vexp + (size_t)(bvr + __popc(bf & ((1u << r) - 1u))) * 64;
      u32x4 sv[4];
      load_sm(r, true, sv);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 ev = *reinterpret_cast<const u32x4*>(ve + g * 16);
        put_bf16(r, true, sv, 2 * g, u32x2{ev.x, ev.y});
        put_bf16(r, true, sv, 2 * g + 1, u32x2{ev.z, ev.w});
      }
    }
  }
}

// The decoder grid: gridDim.x workgroups of W waves; a grid smaller than the units (a decode
// sharing the chip with other work) takes its units in turn, the table built once.
template <int MODE>
__global__ __launch_bounds__(1024) void k_decode_rows(RowDecArgs a) {
  __shared__ uint32_t lut[kRowLut + kRowSec];
  extern __shared__ __align__(16) uint8_t dsh[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  decode_unit<MODE>(a, lut, dsh, (int)blockIdx.x * W + wave, wave, true);
  for (int g = (int)(blockIdx.x + gridDim.x); g * W < a.units; g += (int)gridDim.x)
    decode_unit<MODE>(a, lut, dsh, g * W + wave, wave, false);
}

// Waves a workgroup of k_decode_rows: the fewest rounds of workgroups over the chip, then the
// most compute units busy (the table is built once per workgroup).
static int row_waves(uint32_t stage_words, int64_t units, int lds_wg_max, int lds_cu, int cus) {
  int best_w = 0;
  int64_t best_rounds = INT64_MAX, best_cus = -1;
  for (int W = 16; W >= 1; --W) {
    const int64_t lds = (int64_t)row_buf_area(W) + (int64_t)W * stage_words * 4 + (kRowLut + kRowSec) * 4;
    if (lds > lds_wg_max) continue;
    const int64_t per_cu = std::max<int64_t>(1, lds_cu / lds);
    const int64_t wgs = (units + W - 1) / W;
    const int64_t rounds = (wgs + per_cu * cus - 1) / (per_cu * cus);
    const int64_t used = std::min<int64_t>(cus, (wgs + per_cu - 1) / per_cu);
    if (rounds < best_rounds || (rounds == best_rounds && used > best_cus)) {
      best_w = W;
      best_rounds = rounds;
      best_cus = used;
    }
  }
  return best_w;
}

// 13-bit codes: their 12-bit prefixes (consecutive in a canonical code) each get a block of two
// secondary entries chosen by the 13th bit.  False when they span more prefixes than the
// secondary table holds (then the general decoder takes the matrix).
static bool row_code_prefixes(const uw_info& info, uint32_t* pbase, uint32_t* nblk) {
  uint32_t lo = kRowLut, hi = 0;
  for (int sym = 0; sym < 16; ++sym) {
    const int L = info.code_len[sym];
    if (L > kRowWin) {
      lo = std::min<uint32_t>(lo, (uint32_t)info.code[sym] >> (L - kRowWin));
      hi = std::max<uint32_t>(hi, (uint32_t)info.code[sym] >> (L - kRowWin));
    }
  }
  *pbase = lo;
  *nblk = lo < (uint32_t)kRowLut ? hi - lo + 1 : 0u;
  return *nblk <= (uint32_t)kRowSecBlocks - 1;
}

// The primary table on the host, entry for entry as build_row_lut makes it: the greedy parse
// of each 12-bit window into up to five whole codes.
static void build_row_lut_host(const uw_info& info, uint32_t pbase, uint32_t nblk, uint32_t* lut) {
  uint16_t first[kRowLut];
  std::memset(first, 0, sizeof(first));
  for (int s = 0; s < 16; ++s) {
    const int L = info.code_len[s];
    if (L == 0 || L > kRowWin) continue;
    const uint32_t lo = (uint32_t)info.code[s] << (kRowWin - L), cnt = 1u << (kRowWin - L);
    for (uint32_t i = 0; i < cnt; ++i) first[lo + i] = (uint16_t)(s | (L << 4) | 0x100);
  }
  for (uint32_t w = 0; w < (uint32_t)kRowLut; ++w) {
    if (!(first[w] & 0x100u)) {
      const uint32_t i = w - pbase;
      lut[w] = i < nblk ? (i + 1u) << 9 : 0u;
      continue;
    }
    uint32_t used = (first[w] >> 4) & 15u, n = 1, syms = first[w] & 15u;
    while (n < (uint32_t)kRowMaxSyms) {
      const uint32_t ej = first[(w << used) & (kRowLut - 1)], lj = (ej >> 4) & 15u;
      if (!(ej & 0x100u) || used + lj > (uint32_t)kRowWin) break;
      syms |= (ej & 15u) << (4 * n);
      used += lj;
      ++n;
    }
    lut[w] = (syms << 12) | (4u * n << 4) | used;
  }
}

// Tables built at bind time, one per code, in a per-device array of fixed size (no allocation;
// each GPU holds its copy until the process ends).  The key is the 16 code lengths (the table
// depends on nothing else).  A full cache, or a call on another device than the bind's, leaves
// the kernel to build the table itself, and so does the environment variable
// UW_ROW_TABLE_IN_KERNEL (set to anything; read at every bind and call; for tests of that path).
constexpr int kLutSlots = 128;
static __device__ __align__(256) uint32_t g_row_luts[kLutSlots * kRowLut];
namespace {
struct LutCache {
  std::mutex mu;
  bool init = false;
  uint32_t* base = nullptr;
  int used = 0;
  uint8_t key[kLutSlots][16];
};
LutCache g_lut_cache[64];
}  // namespace

static const uint32_t* row_lut_find(LutCache& c, const uw_info& info) {
  for (int i = 0; i < c.used; ++i)
    if (std::memcmp(c.key[i], info.code_len, 16) == 0) return c.base + (size_t)i * kRowLut;
  return nullptr;
}

static bool row_table_in_kernel() { return std::getenv("UW_ROW_TABLE_IN_KERNEL") != nullptr; }

void register_row_lut(const uw_info& info) {
  if (row_table_in_kernel()) return;
  uint32_t pbase = 0, nblk = 0;
  if (info.chunk / kSeg > 8 || !row_code_prefixes(info, &pbase, &nblk)) return;   // the general decoder's case
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return;
  }
  LutCache& c = g_lut_cache[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  if (!c.init) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_row_luts)) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    c.base = reinterpret_cast<uint32_t*>(p);
    c.init = true;
  }
  if (!c.base || c.used == kLutSlots || row_lut_find(c, info)) return;
  static thread_local uint32_t table[kRowLut];
  build_row_lut_host(info, pbase, nblk, table);
  if (hipMemcpy(c.base + (size_t)c.used * kRowLut, table, sizeof(table), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  std::memcpy(c.key[c.used], info.code_len, 16);
  ++c.used;
}

static const uint32_t* row_lut_lookup(const uw_info& info, int dev) {
  if (dev < 0 || dev >= 64 || row_table_in_kernel()) return nullptr;
  LutCache& c = g_lut_cache[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  return c.base ? row_lut_find(c, info) : nullptr;
}

static uw_status run_decode_rows(const uw_dmat* d, int mode, uint8_t* out, uint32_t* err, int max_wgs, hipStream_t s) {
  RowDecArgs a;
  std::memset(&a, 0, sizeof(a));
  a.words = d->words;
  a.off = d->off;
  a.cbase = d->cbase;
  a.flags = d->flags;
  a.vprefix = d->vprefix;
  a.vexp = d->vexp;
  a.sm = d->sm;
  a.out = out;
  a.err = err;
  a.words_cap = d->words_cap;
  a.n = (int32_t)d->info.n;
  a.k = (int32_t)d->info.k;
  a.kb = (int32_t)d->info.kb;
  a.spc = d->dec_spc;
  a.cpb = d->dec_cpb;
  a.nb = d->dec_nb;
  a.spc_magic = (65536u + (uint32_t)a.spc - 1u) / (uint32_t)a.spc;
  a.units_per_tile = (a.kb + a.nb - 1) / a.nb;
  const int64_t units = (int64_t)d->info.tiles * a.units_per_tile;
  if (units > INT32_MAX) return fail(UW_E_SHAPE, "too many decoder units");
  a.units = (int32_t)units;
  a.stage_words = d->dec_stage_words;
  std::memcpy(a.tab, d->info.palette, 16);
  std::memcpy(a.len, d->info.code_len, 16);
  std::memcpy(a.code, d->info.code, 32);
  for (int sym = 0; sym < 16; ++sym) {
    const uint32_t L = d->info.code_len[sym];
    if (sym < 8) a.len_lo |= L << (4 * sym); else a.len_hi |= L << (4 * (sym - 8));
  }
  if (!row_code_prefixes(d->info, &a.pbase, &a.nblk)) return UW_E_SHAPE;   // the general decoder takes it
  for (int sym = 0; sym < 16; ++sym) {
    const int L = d->info.code_len[sym];
    if (L <= kRowWin) continue;
    if (L != kRowWin + 1) return fail(UW_E_FORMAT, "code length %d exceeds 13", L);
    const uint32_t code = d->info.code[sym], blk = (code >> 1) - a.pbase + 1;
    a.sec[blk * 2 + (code & 1u)] = ((uint32_t)sym << 12) | (4u << 4) | (uint32_t)L;
  }
  static int cache[64][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(UW_E_HIP, "cannot query the device");
  if (!cache[dev][0]) {
    int v[3] = {0, 0, 0};
    if (hipDeviceGetAttribute(&v[0], hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipDeviceGetAttribute(&v[1], hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&v[2], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(UW_E_HIP, "cannot query the LDS size");
    cache[dev][1] = v[0];
    cache[dev][2] = std::max(v[1], v[0]);
    cache[dev][3] = std::max(v[2], 1);
    cache[dev][0] = 1;
  }
  a.lut_src = row_lut_lookup(d->info, dev);
  const int W = row_waves(a.stage_words, units, cache[dev][1], cache[dev][2], cache[dev][3]);
  if (W == 0) return fail(UW_E_SHAPE, "decoder unit needs more LDS than the device allows");
  a.stage_off = row_buf_area(W);
  const size_t lds = (size_t)a.stage_off + (size_t)W * a.stage_words * 4;
  int64_t wgs = (units + W - 1) / W;
  if (max_wgs > 0) wgs = std::min<int64_t>(wgs, max_wgs);
  const dim3 grid((unsigned)wgs);
  switch (mode) {
    case DEC_IDX: hipLaunchKernelGGL(k_decode_rows<DEC_IDX>, grid, dim3(64 * W), lds, s, a); break;
    case DEC_EXP: hipLaunchKernelGGL(k_decode_rows<DEC_EXP>, grid, dim3(64 * W), lds, s, a); break;
    case DEC_BF16: hipLaunchKernelGGL(k_decode_rows<DEC_BF16>, grid, dim3(64 * W), lds, s, a); break;
    default: return fail(UW_E_ARG, "unknown decode target %d", mode);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "decode launch: %s", hipGetErrorString(e));
  return UW_OK;
}

uw_status run_decode(const uw_dmat* d, int mode, uint8_t* out, void* ws, size_t ws_bytes, hipStream_t s, int max_wgs) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!out) return fail(UW_E_ARG, "null output");
  if (!ws || ws_bytes < (size_t)kErrBytes) return fail(UW_E_WORKSPACE, "decode needs a %d-byte workspace", kErrBytes);
  if (d->dec_spc <= 8) {
    // Chunks of at most eight rows: the row decoder, unless the code's 13-bit codes span more
    // prefixes than its secondary table holds (then the general decoder below).
    const uw_status rs = run_decode_rows(d, mode, out, reinterpret_cast<uint32_t*>(ws), max_wgs, s);
    if (rs != UW_E_SHAPE) return rs;
  }
  DecArgs a;
  std::memset(&a, 0, sizeof(a));
  a.words = d->words;
  a.off = d->off;
  a.cbase = d->cbase;
  a.flags = d->flags;
  a.vprefix = d->vprefix;
  a.vexp = d->vexp;
  a.sm = d->sm;
  a.out = out;
  a.err = reinterpret_cast<uint32_t*>(ws);
  a.words_cap = d->words_cap;
  a.n = (int32_t)d->info.n;
  a.k = (int32_t)d->info.k;
  a.kb = (int32_t)d->info.kb;
  a.spc = d->dec_spc;
  a.cpb = d->dec_cpb;
  a.nb = d->dec_nb;
  a.stage_words = d->dec_stage_words;
  std::memcpy(a.tab, d->info.palette, 16);
  std::memcpy(a.len, d->info.code_len, 16);
  std::memcpy(a.code, d->info.code, 32);
  // Codes longer than the lookup window: their 10-bit prefixes (consecutive in a canonical
  // code) each get a block of 8 secondary entries indexed by the next 3 bits.
  for (int i = 0; i < kDecSec; ++i) a.sec[i] = 0;               // count 0: invalid
  a.pbase = kDecLut;
  for (int sym = 0; sym < 16; ++sym) {
    const int L = d->info.code_len[sym];
    if (L > kDecWin) a.pbase = std::min<uint32_t>(a.pbase, (uint32_t)d->info.code[sym] >> (L - kDecWin));
  }
  for (int sym = 0; sym < 16; ++sym) {
    const int L = d->info.code_len[sym];
    if (L <= kDecWin) continue;
    const uint32_t code = d->info.code[sym], pre = code >> (L - kDecWin), blk = pre - a.pbase;
    if (blk >= 15) return fail(UW_E_FORMAT, "long codes span too many prefixes");
    a.pmask |= 1u << blk;
    const uint32_t low = (code << (13 - L)) & 7u, cnt = 1u << (13 - L);
    for (uint32_t q = 0; q < cnt; ++q) a.sec[(blk + 1) * 8 + low + q] = (1u << 29) | ((uint32_t)L << 20) | ((uint32_t)L << 16) | (uint32_t)sym;
  }
  const DecLds L = dec_lds(a.nb, a.stage_words);
  int dev = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return fail(UW_E_HIP, "cannot query the LDS size");
  if (L.total + kDecTableBytes > (uint32_t)lds_max)
    return fail(UW_E_SHAPE, "decoder unit needs %u bytes of LDS (device allows %d)", L.total + kDecTableBytes, lds_max);
  const dim3 grid((unsigned)((d->info.kb + a.nb - 1) / a.nb), (unsigned)d->info.tiles);
  switch (mode) {
    case DEC_IDX: hipLaunchKernelGGL(k_decode<DEC_IDX>, grid, dim3(64), L.total, s, a); break;
    case DEC_EXP: hipLaunchKernelGGL(k_decode<DEC_EXP>, grid, dim3(64), L.total, s, a); break;
    default: hipLaunchKernelGGL(k_decode<DEC_BF16>, grid, dim3(64), L.total, s, a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "decode launch: %s", hipGetErrorString(e));
  return UW_OK;
}

}  // namespace uw
