// libuw device side for MI355X (gfx950): Huffman decoder (to indices, exponents or BF16),
// reconstructive GEMM (palette / exponent / BF16 operand), MLP glue, and the device-facing
// C ABI.
//
// Method: Cloudflare blog post "Unweight".
//  - Reconstructive-matmul paragraphs: compressed weights are read from HBM, BF16 is rebuilt
//    on chip and fed straight to the matrix unit; the rebuilt matrix never reaches HBM.  Here
//    the rebuild happens in VGPRs, directly in the bf16 MFMA operand layout (CDNA MFMA reads
//    its operands from registers, unlike Hopper's shared-memory WGMMA operands).
//  - Rare-exponent paragraph: one decision per 64-weight segment; a verbatim segment swaps the
//    palette lookup for its raw exponent bytes.
//  - SM-split paragraph: the Huffman decoder keeps its lookup table in on-chip memory (here
//    8 KB of LDS: 2^13 one-byte entries, symbol | length << 4).
//  - Four-pipeline paragraphs: decode to BF16 (then a BF16 GEMM), to exponent bytes, or to
//    4-bit indices; direct palette skips the decode.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>

#include "uw_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace uw {

// =========================================================================================
// Reconstruction helpers.  A bf16 pair register holds weight 2j in bits 0..15 and weight
// 2j+1 in bits 16..31 (the MFMA operand element order).
//   pair = (spread(sm) & 0x807F807F) | (E_lo << 7) | (E_hi << 23)
// where spread(sm) = [sm_lo, sm_lo, sm_hi, sm_hi] bytes puts each sign bit at bit 15 of its
// half and each mantissa at bits 6..0.
// =========================================================================================
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Sign+mantissa dwords (4 weights each) -> 4 spread pair words.
__device__ __forceinline__ void spread_sm(uint32_t s_lo, uint32_t s_hi, uint32_t p[4]) {
  p[0] = perm(s_lo, s_lo, 0x01010000u);
  p[1] = perm(s_lo, s_lo, 0x03030202u);
  p[2] = perm(s_hi, s_hi, 0x01010000u);
  p[3] = perm(s_hi, s_hi, 0x03030202u);
}

// Affine palette (palette[i] = palette[0] + i): an index word holds the 8 indices of one
// MFMA step, weight 2j at bits 4j and weight 2j+1 at bits 16+4j, so each pair's two
// exponents are one mask and one shift-add away.  base2 = p0 << 7 | p0 << 23.
// m0 = 0x000F000F and m1 = 0x00F000F0 arrive as kernel arguments: with the masks opaque
// the compiler keeps "mask, then shift-add" (v_and + v_lshl_add) instead of rewriting it into
// shift, mask, add.
__device__ __forceinline__ void exps_affine(uint32_t iw, uint32_t base2, uint32_t m0, uint32_t m1, uint32_t T[4]) {
  T[0] = ((iw & m0) << 7) + base2;
  T[1] = ((iw & m1) << 3) + base2;
  const uint32_t h = iw >> 8;
  T[2] = ((h & m0) << 7) + base2;
  T[3] = ((h & m1) << 3) + base2;
}

// Byte-wise lookup of 4 indices (0..15, one per byte of sel) in a 16-byte table held in
// four registers: two 8-entry byte permutes and a byte select on bit 3.
__device__ __forceinline__ uint32_t lookup16(uint32_t sel, const uint32_t tab[4]) {
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t lo = perm(tab[1], tab[0], s7);
  const uint32_t hi = perm(tab[3], tab[2], s7);
  const uint32_t t = (sel >> 3) & 0x01010101u;
  const uint32_t m = (t << 8) - t;  // 0xFF in every byte whose index is >= 8
  return (hi & m) | (lo & ~m);
}

// General palette: exponents by table lookup, then placed at bits 7 and 23 of each pair.
__device__ __forceinline__ void exps_lut(uint32_t iw, const uint32_t tab[4], uint32_t T[4]) {
  const uint32_t e04 = lookup16(iw & 0x0F0F0F0Fu, tab);          // bytes: E0 E4 E1 E5
  const uint32_t e26 = lookup16((iw >> 4) & 0x0F0F0F0Fu, tab);   // bytes: E2 E6 E3 E7
  T[0] = (e04 & 0x00FF00FFu) << 7;
  T[2] = (e04 & 0xFF00FF00u) >> 1;
  T[1] = (e26 & 0x00FF00FFu) << 7;
  T[3] = (e26 & 0xFF00FF00u) >> 1;
}

// Raw exponent bytes (4 per dword) -> pair exponent words.
__device__ __forceinline__ void exps_raw(uint32_t e_lo, uint32_t e_hi, uint32_t T[4]) {
  T[0] = perm(e_lo, e_lo, 0x0C010C00u) << 7;
  T[1] = perm(e_lo, e_lo, 0x0C030C02u) << 7;
  T[2] = perm(e_hi, e_hi, 0x0C010C00u) << 7;
  T[3] = perm(e_hi, e_hi, 0x0C030C02u) << 7;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// =========================================================================================
// Reconstructive GEMM.
//
// Work split: one workgroup per 16-row tile (grid.x), all M columns in CT MFMA column tiles
// of 16 (grid.y covers M beyond 16*CT).  The workgroup's waves split the tile's 64-column
// blocks into contiguous ranges and their partial 16x16 accumulators are summed in LDS in a
// fixed order (deterministic).
// Per block a lane (row r = lane%16, column group g = lane/16) owns 16 consecutive weights:
// 16 sign+mantissa bytes at lane*16 of the block's 1 KB (one dwordx4, the whole wave reads
// 1 KB contiguously) and 8 index bytes at lane*8 of its 512 B.  MFMA step s = 0, 1 takes the
// lane's weights 8s..8s+7 for A and X[m][64b + 16g + 8s .. +8] for B; any k-permutation that
// A and B share leaves the dot product unchanged.
// =========================================================================================
enum Src { SRC_PAL_AFFINE = 0, SRC_PAL_LUT = 1, SRC_EXP = 2, SRC_BF16 = 3 };

struct GemmArgs {
  const uint8_t* sm;        // sign+mantissa sub-tiles (palette / exponent sources)
  const uint8_t* aux;       // index stream | exponent sub-tiles | BF16 W row-major
  const uint16_t* flags;
  const uint32_t* vprefix;
  const uint8_t* vexp;
  const uint16_t* x;
  float* y;
  int32_t n, k, m, kb;
  uint32_t base2;
  uint32_t tab[4];
  uint32_t m0, m1;  // 0x000F000F, 0x00F000F0 (see exps_affine)
};

template <int SRC>
struct WRegs;
template <>
struct WRegs<SRC_PAL_AFFINE> { u32x4 s; u32x2 i; };
template <>
struct WRegs<SRC_PAL_LUT> { u32x4 s; u32x2 i; };
template <>
struct WRegs<SRC_EXP> { u32x4 s; u32x4 e; };
template <>
struct WRegs<SRC_BF16> { u32x4 w0, w1; };

// Raw buffer loads (bounds-checked): a lane whose offset is past num_records receives zeros
// and generates no memory traffic.  That lets every load of the steady-state loop be an
// unconditional instruction (exact in-order vmcnt waits) while only the lanes that need X
// rows or verbatim exponents fetch them.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, 0));
}
// Streaming (read-once) weight loads: the nontemporal cache policy bit.
constexpr int kNt = 2;
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, kNt));
}
__device__ __forceinline__ u32x2 bload8_nt(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, kNt));
}

// One prefetch slot: everything block b's compute needs from global memory, so compute
// issues no global load (global loads retire in order: a load issued inside compute would
// also wait for every prefetched block behind it).  X rows (XL) and verbatim exponents (VS)
// can instead come from LDS, which keeps the slot at 6 VGPRs for the palette source.
template <int SRC, int CT, int XL, int VS>
struct Slot {
  WRegs<SRC> w;
  u32x4 xb0[XL ? 1 : CT], xb1[XL ? 1 : CT];  // B operand from global (zeros past the valid rows)
  u32x4 ev;                                   // VS == 0: this lane's verbatim exponents
};

template <int CT, int U>
struct MaxThreads { static constexpr int v = CT == 1 ? (U >= 8 ? 512 : 1024) : (CT == 2 ? 512 : 256); };
static inline int max_waves(int ct, int unroll) { return ct == 1 ? (unroll >= 8 ? 8 : 16) : ct == 2 ? 8 : 4; }

__host__ __device__ constexpr int xl_stride(int k) { return 2 * k + 16; }  // padded X row in LDS
constexpr int kVexpStageSegs = 256;  // VS: up to this many verbatim segments per tile in LDS (16 KB)
constexpr int kXlMaxBytes = 48 * 1024;

// Global -> LDS staging with LDS-DMA buffer loads (no VGPRs: the data goes straight to LDS;
// lane i of one instruction writes `size` bytes at lds + i*size).  Out-of-range lanes write
// zeros.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// LDS layout of k_gemm (bytes): partial sums | flags (u16) | verbatim prefix (u32) |
// verbatim exponents | X rows (padded) + one zero row.
struct LdsLayout {
  uint32_t red, fl, vp, ve, x, total;
};
__host__ __device__ inline LdsLayout lds_layout(int nw, int ct, int kb, bool pal, bool vs, bool xl, int mv, int k) {
  LdsLayout L;
  L.red = 0;
  L.fl = (uint32_t)nw * ct * 64 * 16;
  L.vp = L.fl + (pal ? (uint32_t)((kb * 2 + 15) / 16 * 16) : 0u);
  L.ve = L.vp + (pal ? (uint32_t)(((kb + 1) * 4 + 15) / 16 * 16) : 0u);
  L.x = L.ve + (pal && vs ? (uint32_t)kVexpStageSegs * 64 : 0u);
  L.total = L.x + (xl ? (uint32_t)(mv + 1) * xl_stride(k) : 0u);
  return L;
}

// Dynamic LDS: [nw*CT*64 floatx4 partial sums][kb u32 flags][kb+1 u32 verbatim prefix]
//              [VS: staged verbatim exponents][XL: mv padded X rows + 1 zero row]
template <int SRC, int CT, int U, int XL, int VS>
__global__ __launch_bounds__((MaxThreads<CT, U>::v)) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int t = blockIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int kb = a.kb;
  const int b0 = (int)((int64_t)wave * kb / nw), b1 = (int)((int64_t)(wave + 1) * kb / nw);
  const int nblk = b1 - b0;  // >= 1: the launcher keeps nw <= kb
  const int mcol0 = blockIdx.y * 16 * CT;
  const int mv = min(16 * CT, a.m - mcol0);  // valid X rows of this column block
  constexpr bool kPal = SRC <= SRC_PAL_LUT;
  const LdsLayout lay = lds_layout(nw, CT, kb, kPal, VS, XL, mv, a.k);
  floatx4* red = reinterpret_cast<floatx4*>(smem + lay.red);
  uint16_t* sfl = reinterpret_cast<uint16_t*>(smem + lay.fl);
  uint32_t* svp = reinterpret_cast<uint32_t*>(smem + lay.vp);
  uint8_t* sve = smem + lay.ve;
  uint8_t* sx = smem + lay.x;

  floatx4 acc[CT], acc2[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc2[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // Weight streams through buffer resources based at this tile: the per-lane offset is fixed
  // and the block offset goes in soffset, so a load costs no address VGPRs.
  const size_t tile_bytes = (size_t)t * a.k * 16;
  const int row = t * 16 + r;
  const bool row_ok = row < a.n;
  __amdgpu_buffer_rsrc_t wrs0, wrs1;
  uint32_t woff0, woff1;
  if constexpr (SRC == SRC_BF16) {
    const int rows = min(16, a.n - t * 16);
    wrs0 = make_rsrc(a.aux + tile_bytes * 2, (uint32_t)rows * a.k * 2);  // rows past n read zeros
    wrs1 = wrs0;
    woff0 = row_ok ? (uint32_t)(r * a.k + g * 16) * 2 : kOob;
    woff1 = 0;
  } else {
    wrs0 = make_rsrc(a.sm + tile_bytes, (uint32_t)a.k * 16);
    woff0 = lane * 16;
    if constexpr (SRC == SRC_EXP) {
      wrs1 = make_rsrc(a.aux + tile_bytes, (uint32_t)a.k * 16);
      woff1 = lane * 16;
    } else {
      wrs1 = make_rsrc(a.aux + tile_bytes / 2, (uint32_t)a.k * 8);
      woff1 = lane * 8;
    }
  }
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (size_t)mcol0 * a.k, (uint32_t)mv * a.k * 2);
  uint32_t xoff[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) xoff[c] = 16 * c + r < mv ? (uint32_t)((16 * c + r) * a.k + g * 16) * 2 : kOob;
  // XL: LDS byte offset of this lane's X row; rows past mv read the zero row after the X rows
  const uint32_t xl_off = (uint32_t)((r < mv ? r : mv) * xl_stride(a.k) + g * 32);

  uint32_t vbase = 0;
  __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vexp, 0);

  // Loads of block b; `ok` false turns every lane offset out of range (zeros, no traffic), so
  // a batch's loads are unconditional instructions even past the wave's last block.
  auto load_main = [&](int b, bool ok, Slot<SRC, CT, XL, VS>& sl) {
    const uint32_t o0 = ok ? woff0 : kOob;
    if constexpr (SRC == SRC_BF16) {
      sl.w.w0 = bload16_nt(wrs0, o0, b * 128);
      sl.w.w1 = bload16_nt(wrs0, o0 == kOob ? kOob : o0 + 16, b * 128);
    } else if constexpr (SRC == SRC_EXP) {
      sl.w.s = bload16_nt(wrs0, o0, b * 1024);
      sl.w.e = bload16_nt(wrs1, ok ? woff1 : kOob, b * 1024);
    } else {
      sl.w.s = bload16_nt(wrs0, o0, b * 1024);
      sl.w.i = bload8_nt(wrs1, ok ? woff1 : kOob, b * 512);
    }
    if constexpr (!XL) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const uint32_t o = (xoff[c] == kOob || !ok) ? kOob : xoff[c] + b * 128;
        sl.xb0[c] = bload16(xrs, o);
        sl.xb1[c] = bload16(xrs, o == kOob ? kOob : o + 16);
      }
    }
  };
  // VS == 0: verbatim exponents through the ring (bounds-checked load, zeros unless flagged).
  auto load_ev = [&](int b, Slot<SRC, CT, XL, VS>& sl) {
    if constexpr (kPal && !VS) {
      const uint32_t f = __builtin_amdgcn_readfirstlane(sfl[b]);
      const uint32_t rank = __builtin_amdgcn_readfirstlane(svp[b]) + __popc(f & ((1u << r) - 1u));
      sl.ev = bload16(vrs, ((f >> r) & 1u) ? rank * 64 + g * 16 : kOob);
    }
  };

  // Per-wave copies of the tile's flags / verbatim prefixes, block b0 + j in lane j (the
  // launcher keeps every wave's range within 64 blocks), filled after the LDS staging.
  uint32_t wfl = 0, wvp = 0;
  auto wave_flag = [&](int b) -> uint32_t { return __builtin_amdgcn_readlane(wfl, b - b0); };
  auto wave_vpre = [&](int b) -> uint32_t { return __builtin_amdgcn_readlane(wvp, b - b0); };

  auto compute = [&](int b, const Slot<SRC, CT, XL, VS>& sl) {
    u32x4 A0, A1;
    if constexpr (SRC == SRC_BF16) {
      A0 = sl.w.w0;  // rows past n arrive as zeros (bounds-checked load)
      A1 = sl.w.w1;
    } else {
      uint32_t T0[4], T1[4];
      if constexpr (SRC == SRC_PAL_AFFINE) {
        exps_affine(sl.w.i.x, a.base2, a.m0, a.m1, T0);
        exps_affine(sl.w.i.y, a.base2, a.m0, a.m1, T1);
      } else if constexpr (SRC == SRC_PAL_LUT) {
        exps_lut(sl.w.i.x, a.tab, T0);
        exps_lut(sl.w.i.y, a.tab, T1);
      } else {
        exps_raw(sl.w.e.x, sl.w.e.y, T0);
        exps_raw(sl.w.e.z, sl.w.e.w, T1);
      }
      if constexpr (kPal) {
        // This wave's flags and verbatim prefixes sit one block per lane in wfl / wvp.
        const uint32_t f = wave_flag(b);
        if (f) {  // uniform: some row of this tile has a verbatim segment in block b
          const bool mine = (f >> r) & 1u;
          u32x4 ev;
          if constexpr (VS) {
            const uint32_t rank = wave_vpre(b) + __popc(f & ((1u << r) - 1u));
            ev = *reinterpret_cast<const u32x4*>(sve + (mine ? rank * 64 + g * 16 : 0u));
          } else {
            ev = sl.ev;
          }
          uint32_t R0[4], R1[4];
          exps_raw(ev.x, ev.y, R0);
          exps_raw(ev.z, ev.w, R1);
          const uint32_t keep = mine ? 0u : ~0u;  // element-wise select, no array select
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            T0[j] = (T0[j] & keep) | (R0[j] & ~keep);
            T1[j] = (T1[j] & keep) | (R1[j] & ~keep);
          }
        }
      }
      uint32_t P0[4], P1[4];
      spread_sm(sl.w.s.x, sl.w.s.y, P0);
      spread_sm(sl.w.s.z, sl.w.s.w, P1);
      A0 = u32x4{(P0[0] & 0x807F807Fu) | T0[0], (P0[1] & 0x807F807Fu) | T0[1], (P0[2] & 0x807F807Fu) | T0[2],
                 (P0[3] & 0x807F807Fu) | T0[3]};
      A1 = u32x4{(P1[0] & 0x807F807Fu) | T1[0], (P1[1] & 0x807F807Fu) | T1[1], (P1[2] & 0x807F807Fu) | T1[2],
                 (P1[3] & 0x807F807Fu) | T1[3]};
    }
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, A0), a1 = __builtin_bit_cast(bf16x8, A1);
    // Two accumulator sets (MFMA step 0 and step 1) so consecutive MFMAs do not depend on
    // each other; summed in the epilogue.
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      u32x4 x0, x1;
      if constexpr (XL) {  // X rows from LDS (rows past mv read the zero row)
        const u32x4* xp = reinterpret_cast<const u32x4*>(sx + xl_off + b * 128);
        x0 = xp[0];
        x1 = xp[1];
      } else {
        x0 = sl.xb0[c];
        x1 = sl.xb1[c];
      }
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, x0), acc[c], 0, 0, 0);
      acc2[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, x1), acc2[c], 0, 0, 0);
    }
  };

  // Schedule: the wave's blocks go in batches of U.  A batch issues all its loads, then
  // computes its blocks; nothing is carried in registers from one batch to the next, so the
  // waits are exact and no copy ever waits on a load.  Memory latency is covered by the U
  // loads of a batch and by the other waves on the SIMD.
  // Prologue: the LDS staging loads (flags, verbatim exponents, X rows) go out first, then the
  // first batch; staging data returns first (loads retire in order), so the barriers below
  // do not wait for the batch.
  Slot<SRC, CT, XL, VS> buf[U];
  uint16_t stf[4];
  if constexpr (kPal) {
    vbase = a.vprefix[t];
    const uint32_t nvt = a.vprefix[t + 1] - vbase;
    vrs = make_rsrc(a.vexp + (size_t)vbase * 64, nvt * 64);
    const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.flags + (size_t)t * kb, (uint32_t)kb * 2);
    // Flags: up to 4 bounds-checked 16-bit loads a thread (sub-dword LDS-DMA would not pack
    // them), stored to LDS once they arrive; a longer tile row takes the loop below.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      stf[j] = __builtin_amdgcn_raw_buffer_load_b16(frs, i < kb ? (uint32_t)i * 2 : kOob, 0, 0);
    }
    if constexpr (VS)
      for (int c = wave; c * 16 < (int)nvt; c += nw) lds_dma16(vrs, sve + c * 1024, (uint32_t)c * 1024 + lane * 16);
  }
  if constexpr (XL) {  // X rows, 1 KB a DMA (the launcher requires k % 512 == 0)
    const int per_row = a.k / 512;
    for (int c = wave; c < mv * per_row; c += nw) {
      const int mr = c / per_row, cc = c - mr * per_row;
      lds_dma16(xrs, sx + (size_t)mr * xl_stride(a.k) + cc * 1024, (uint32_t)mr * a.k * 2 + cc * 1024 + lane * 16);
    }
    for (int i = threadIdx.x; i < xl_stride(a.k) / 16; i += blockDim.x)
      reinterpret_cast<u32x4*>(sx + (size_t)mv * xl_stride(a.k))[i] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) load_main(b0 + u, u < nblk, buf[u]);
  if constexpr (kPal) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      if (i < kb) sfl[i] = stf[j];
    }
    for (int i = threadIdx.x + 4 * blockDim.x; i < kb; i += blockDim.x) sfl[i] = a.flags[(size_t)t * kb + i];
  }
  if constexpr (kPal || XL) __syncthreads();
  if constexpr (kPal) {
    if (wave == 0) {  // exclusive prefix of verbatim counts per block (wave-level scan)
      uint32_t carry = 0;
      for (int j = 0; j < kb; j += 64) {
        const int b = j + lane;
        const uint32_t v = b < kb ? (uint32_t)__popc((uint32_t)sfl[b]) : 0u;
        const uint32_t incl = wave_incl_scan(v, lane);
        if (b < kb) svp[b] = carry + incl - v;
        carry += __shfl(incl, 63, 64);
      }
    }
    __syncthreads();
    wfl = b0 + lane < kb ? sfl[b0 + lane] : 0u;
    wvp = b0 + lane < kb ? svp[b0 + lane] : 0u;
  }
  auto run_batch = [&](int b) {
    if constexpr (kPal && !VS) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b + u < b1) load_ev(b + u, buf[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u < b1) compute(b + u, buf[u]);
  };
  run_batch(b0);
  for (int b = b0 + U; b < b1; b += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_main(b + u, b + u < b1, buf[u]);
    run_batch(b);
  }

#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] += acc2[c];
  // Epilogue: D lane layout = column m (lane%16), rows 4*(lane/16) + j.
  auto store = [&](int c, int l, floatx4 v) {
    const int mm = mcol0 + 16 * c + (l & 15);
    if (mm >= a.m) return;
    const int n0 = t * 16 + 4 * (l >> 4);
    float* yp = a.y + (size_t)mm * a.n + n0;
    if (n0 + 3 < a.n && (a.n & 3) == 0) {
      *reinterpret_cast<floatx4*>(yp) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.n) yp[j] = v[j];
    }
  };
  if (nw == 1) {
#pragma unroll
    for (int c = 0; c < CT; ++c) store(c, lane, acc[c]);
    return;
  }
#pragma unroll
  for (int c = 0; c < CT; ++c) red[(wave * CT + c) * 64 + lane] = acc[c];
  __syncthreads();
  for (int s = threadIdx.x; s < CT * 64; s += blockDim.x) {
    floatx4 v = red[s];
    for (int w = 1; w < nw; ++w) v += red[w * CT * 64 + s];
    store(s >> 6, s & 63, v);
  }
}

// =========================================================================================
// Huffman decoder.
//
// One workgroup (one wave) per (tile, group of 64 chunks); lane i decodes chunk
// cbase[t] + 64*part + i serially.  Chunks restart at every tile and cover whole segments,
// so a lane places its output from the tile's verbatim flags alone: a wave-level prefix sum
// of per-block verbatim counts (LDS) gives each block's first coded-segment rank, a binary
// search finds the chunk's first segment, and the lane then walks forward, skipping verbatim
// rows.  Workgroup part 0 also writes the verbatim segments and the padding rows.
// =========================================================================================
enum DecMode { DEC_IDX = 0, DEC_EXP = 1, DEC_BF16 = 2 };

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
  int32_t n, k, kb, chunk;
  uint8_t pal[16];
  uint8_t len[16];
  uint16_t code[16];
};

struct BitReader {
  const uint32_t* words;
  uint32_t cap;
  u32x4 qa, qb;   // words [base, base+4) and [base+4, base+8)
  uint32_t base;
  int ci;         // next word of qa to hand out
  uint64_t buf;   // stream bits, left aligned
  int avail;      // valid bits in buf
  uint32_t pos;   // stream position of buf's top bit

  __device__ __forceinline__ u32x4 load4(uint32_t i) const {
    if (i + 4 <= cap) return *reinterpret_cast<const u32x4*>(words + i);
    u32x4 v = {0, 0, 0, 0};
    if (i < cap) v.x = words[i];
    if (i + 1 < cap) v.y = words[i + 1];
    if (i + 2 < cap) v.z = words[i + 2];
    if (i + 3 < cap) v.w = words[i + 3];
    return v;
  }
  __device__ __forceinline__ uint32_t take() {
    const uint32_t v = ci == 0 ? qa.x : ci == 1 ? qa.y : ci == 2 ? qa.z : qa.w;
    if (++ci == 4) {
      qa = qb;
      base += 4;
      qb = load4(base + 4);
      ci = 0;
    }
    return v;
  }
  __device__ __forceinline__ void init(uint32_t bit) {
    const uint32_t wi = bit >> 5;
    base = wi & ~3u;
    qa = load4(base);
    qb = load4(base + 4);
    ci = (int)(wi - base);
    const uint64_t hi = take(), lo = take();
    const int o = (int)(bit & 31);
    buf = ((hi << 32) | lo) << o;
    avail = 64 - o;
    pos = bit;
  }
  // Next symbol via the 2^13-entry table; returns -1 on an invalid code.
  __device__ __forceinline__ int next(const uint8_t* lut) {
    const uint32_t e = lut[(uint32_t)(buf >> 51)];
    const int L = (int)(e >> 4);
    buf <<= L;
    avail -= L;
    pos += (uint32_t)L;
    if (avail < 32) {
      buf |= (uint64_t)take() << (32 - avail);
      avail += 32;
    }
    return L ? (int)(e & 15u) : -1;
  }
};

__device__ __forceinline__ uint32_t bf16_pairs_from(uint32_t s, uint32_t e, int half) {
  // s, e: 4 sign+mantissa bytes and 4 exponent bytes; half 0 -> weights 0,1; 1 -> 2,3.
  const uint32_t sp = perm(s, s, half ? 0x03030202u : 0x01010000u);
  const uint32_t ep = perm(e, e, half ? 0x0C030C02u : 0x0C010C00u) << 7;
  return (sp & 0x807F807Fu) | ep;
}

template <int MODE>
__device__ __forceinline__ void write_segment(const DecArgs& a, int t, int b, int r, int g, const uint32_t v[4],
                                              bool zero) {
  // v: for DEC_IDX two nibble words in v[0..1]; otherwise 16 exponent bytes in v[0..3].
  const size_t sub = ((size_t)t * (a.k / 16) + 4 * b + g) * 16 + r;
  if constexpr (MODE == DEC_IDX) {
    u32x2 o = zero ? u32x2{0, 0} : u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(a.out + sub * 8) = o;
  } else if constexpr (MODE == DEC_EXP) {
    u32x4 o = zero ? u32x4{0, 0, 0, 0} : u32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<u32x4*>(a.out + sub * 16) = o;
  } else {
    const u32x4 s = *reinterpret_cast<const u32x4*>(a.sm + sub * 16);
    const uint32_t ss[4] = {s.x, s.y, s.z, s.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = bf16_pairs_from(ss[q], v[q], 0);
      o[2 * q + 1] = bf16_pairs_from(ss[q], v[q], 1);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.out + ((size_t)(t * 16 + r) * a.k + 64 * b + 16 * g) * 2);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  }
}

template <int MODE>
__global__ __launch_bounds__(64) void k_decode(DecArgs a) {
  __shared__ uint8_t lut[1 << kLmax];
  __shared__ uint32_t vpre[kMaxK / kSeg + 1];
  const int t = blockIdx.x, part = blockIdx.y, lane = threadIdx.x;
  const int rows = min(16, a.n - 16 * t);
  const uint32_t realmask = rows == 16 ? 0xFFFFu : ((1u << rows) - 1u);
  const uint16_t* flg = a.flags + (size_t)t * a.kb;

  for (int i = lane; i < (1 << kLmax) / 4; i += 64) reinterpret_cast<uint32_t*>(lut)[i] = 0;
  __syncthreads();
  for (int s = 0; s < 16; ++s) {
    const int L = a.len[s];
    if (!L) continue;
    const uint32_t lo = (uint32_t)a.code[s] << (kLmax - L), cnt = 1u << (kLmax - L);
    for (uint32_t i = lane; i < cnt; i += 64) lut[lo + i] = (uint8_t)(s | (L << 4));
  }
  // Exclusive prefix of verbatim segments per block (wave-level scan, 64 blocks a step).
  uint32_t carry = 0;
  for (int base = 0; base < a.kb; base += 64) {
    const int b = base + lane;
    const uint32_t v = b < a.kb ? (uint32_t)__popc(flg[b]) : 0u;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (b < a.kb) vpre[b] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) vpre[a.kb] = carry;
  __syncthreads();

  const uint32_t c0 = a.cbase[t], c1 = a.cbase[t + 1];
  const uint32_t c = c0 + (uint32_t)part * 64 + lane;
  if (c < c1) {
    const uint32_t nsym_tile = ((uint32_t)rows * a.kb - carry) * 64;
    const uint32_t ci = c - c0;
    const uint32_t nseg = min((uint32_t)a.chunk, nsym_tile - ci * a.chunk) / 64;
    const uint32_t q = ci * (uint32_t)(a.chunk / 64);
    // last block b with coded-before(b) = rows*b - vpre[b] <= q
    int lo = 0, hi = a.kb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((uint32_t)rows * mid - vpre[mid] <= q) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    uint32_t cm = realmask & ~(uint32_t)flg[b];
    for (uint32_t j = q - ((uint32_t)rows * b - vpre[b]); j > 0; --j) cm &= cm - 1;
    int r = __ffs(cm) - 1;

    BitReader br;
    br.words = a.words;
    br.cap = a.words_cap;
    br.init(a.off[c]);
    bool bad = false;
    for (uint32_t sgi = 0; sgi < nseg && !bad; ++sgi) {
      for (int g = 0; g < 4; ++g) {
        uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sym = br.next(lut);
          if (sym < 0) bad = true;
          const uint32_t s = (uint32_t)sym & 15u;
          if constexpr (MODE == DEC_IDX) {
            const int ii = i & 7;
            v[i >> 3] |= s << (4 * (ii >> 1) + 16 * (ii & 1));
          } else {
            v[i >> 2] |= (uint32_t)a.pal[s] << (8 * (i & 3));
          }
        }
        write_segment<MODE>(a, t, b, r, g, v, false);
      }
      uint32_t m2 = realmask & ~(uint32_t)flg[b] & ~((2u << r) - 1u);
      while (!m2 && b + 1 < a.kb) {
        ++b;
        m2 = realmask & ~(uint32_t)flg[b];
      }
      r = m2 ? __ffs(m2) - 1 : 0;
    }
    if (bad || br.pos != a.off[c + 1]) atomicOr(a.err, 1u);
  }

  if (part == 0) {
    const uint32_t vt = a.vprefix[t];
    const uint32_t zero4[4] = {0, 0, 0, 0};
    for (int b = lane; b < a.kb; b += 64) {
      const uint32_t f = flg[b];
      uint32_t vr = vt + vpre[b];
      for (int rr = 0; rr < 16; ++rr) {
        if (rr < rows && ((f >> rr) & 1u)) {
          const u32x4* src = reinterpret_cast<const u32x4*>(a.vexp + (size_t)vr * 64);
          ++vr;
          for (int g = 0; g < 4; ++g) {
            const u32x4 e = src[g];
            const uint32_t v[4] = {e.x, e.y, e.z, e.w};
            write_segment<MODE>(a, t, b, rr, g, v, MODE == DEC_IDX);
          }
        } else if (rr >= rows && MODE != DEC_BF16) {
          for (int g = 0; g < 4; ++g) write_segment<MODE>(a, t, b, rr, g, zero4, true);
        }
      }
    }
  }
}

// =========================================================================================
// MLP glue (SwiGLU between up/gate and down; RMS norm feeding the next layer)
// =========================================================================================
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ void k_swiglu(const float* g, const float* u, uint16_t* h, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
    const float gv = g[i];
    h[i] = f32_to_bf16(gv / (1.0f + expf(-gv)) * u[i]);
  }
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float* y, uint16_t* x, int n, float eps) {
  __shared__ float part[4];
  const float* yr = y + (size_t)blockIdx.x * n;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) ss += yr[i] * yr[i];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float scale = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += 256) x[(size_t)blockIdx.x * n + i] = f32_to_bf16(yr[i] * scale);
}

// =========================================================================================
// Host launchers
// =========================================================================================
struct Variant {
  int waves;
  int unroll;
};
static const Variant kVariants[] = {{4, 8}, {2, 8}, {8, 8}, {16, 8}, {1, 8}, {4, 4}, {2, 4}, {8, 4}, {16, 4}, {1, 4}};
static constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

static int col_tiles(int m) {
  const int ct = (m + 15) / 16;
  return ct <= 1 ? 1 : ct <= 2 ? 2 : ct <= 4 ? 4 : 8;
}

static int default_variant(int64_t tiles, int64_t kb, int ct) {
  // Measured on MI355X: about 2048 waves over the chip (8 per CU, all resident at once) with
  // 4-block batches is best for M <= 16; wider M keeps 4-block batches and fewer waves.
  const int cap = ct == 1 ? 16 : ct == 2 ? 8 : 4;
  int w = 1;
  while (w < cap && tiles * w < 1536 && kb / (w * 2) >= 4) w *= 2;
  for (int v = 0; v < kNumVariants; ++v)
    if (kVariants[v].waves == w && kVariants[v].unroll == 4) return v;
  return 0;
}

struct Launch {
  int tiles, waves, unroll;
  int max_tile_verb;  // most verbatim segments in one tile (LDS staging when they all fit)
};

template <int SRC, int CT, int U, int XL, int VS>
static hipError_t launch_gemm_t(const GemmArgs& a, const Launch& L, hipStream_t s) {
  const int gy = (a.m + 16 * CT - 1) / (16 * CT);
  const size_t shm = lds_layout(L.waves, CT, a.kb, SRC <= SRC_PAL_LUT, VS, XL, std::min(a.m, 16 * CT), a.k).total;
  hipLaunchKernelGGL((k_gemm<SRC, CT, U, XL, VS>), dim3(L.tiles, gy), dim3(64 * L.waves), shm, s, a);
  return hipGetLastError();
}

template <int SRC, int CT, int XL, int VS>
static hipError_t launch_gemm_u(const GemmArgs& a, const Launch& L, hipStream_t s) {
  // Deeper prefetch only where the slot stays small enough to avoid spills (X from LDS).
  if constexpr (CT == 1) {
    if (L.unroll >= 8) return launch_gemm_t<SRC, 1, 8, XL, VS>(a, L, s);
    return launch_gemm_t<SRC, 1, 4, XL, VS>(a, L, s);
  } else {
    return launch_gemm_t<SRC, CT, 4, 0, VS>(a, L, s);
  }
}

template <int SRC, int CT>
static hipError_t launch_gemm_v(const GemmArgs& a, const Launch& L, hipStream_t s) {
  constexpr bool pal = SRC <= SRC_PAL_LUT;
  const int mv = std::min(a.m, 16);
  const bool xl = CT == 1 && a.k % 512 == 0 && (size_t)(mv + 1) * xl_stride(a.k) <= (size_t)kXlMaxBytes;
  const bool vs_ok = L.max_tile_verb <= kVexpStageSegs;
  if (pal && vs_ok) return xl ? launch_gemm_u<SRC, CT, CT == 1, 1>(a, L, s) : launch_gemm_u<SRC, CT, 0, 1>(a, L, s);
  return xl ? launch_gemm_u<SRC, CT, CT == 1, 0>(a, L, s) : launch_gemm_u<SRC, CT, 0, 0>(a, L, s);
}

template <int SRC>
static hipError_t launch_gemm_c(const GemmArgs& a, int ct, const Launch& L, hipStream_t s) {
  switch (ct) {
    case 1: return launch_gemm_v<SRC, 1>(a, L, s);
    case 2: return launch_gemm_v<SRC, 2>(a, L, s);
    case 4: return launch_gemm_v<SRC, 4>(a, L, s);
    default: return launch_gemm_v<SRC, 8>(a, L, s);
  }
}

static uw_status run_gemm(int src, const GemmArgs& a, int64_t tiles, int variant, int max_tile_verb, hipStream_t s) {
  int ct = col_tiles(a.m);
  if (variant < 0) variant = default_variant(tiles, a.kb, ct);
  Launch L;
  L.tiles = (int)tiles;
  L.unroll = kVariants[variant].unroll;
  L.max_tile_verb = max_tile_verb;
  // Every wave's block range must fit one lane per block (<= 64 blocks).  Wider column tiles
  // and deeper batches allow fewer waves per workgroup; past that, use shallower batches and
  // 16-column tiles.
  const int need = (a.kb + 63) / 64;
  if (max_waves(ct, L.unroll) < need) L.unroll = 4;
  while (ct > 1 && max_waves(ct, L.unroll) < need) ct >>= 1;
  if (max_waves(ct, L.unroll) < need) return fail(UW_E_SHAPE, "k=%d is too long for this kernel", a.k);
  L.waves = std::min(std::max(kVariants[variant].waves, need), max_waves(ct, L.unroll));
  while (L.waves > 1 && L.waves > a.kb) L.waves >>= 1;
  hipError_t e;
  switch (src) {
    case SRC_PAL_AFFINE: e = launch_gemm_c<SRC_PAL_AFFINE>(a, ct, L, s); break;
    case SRC_PAL_LUT: e = launch_gemm_c<SRC_PAL_LUT>(a, ct, L, s); break;
    case SRC_EXP: e = launch_gemm_c<SRC_EXP>(a, ct, L, s); break;
    default: e = launch_gemm_c<SRC_BF16>(a, ct, L, s); break;
  }
  if (e != hipSuccess) return fail(UW_E_HIP, "gemm launch: %s", hipGetErrorString(e));
  return UW_OK;
}

static uw_status check_dmat(const uw_dmat* d) {
  if (!d || d->magic != kDmatMagic) return fail(UW_E_ARG, "matrix view is not bound");
  return UW_OK;
}

static uw_status run_decode(const uw_dmat* d, int mode, uint8_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!out) return fail(UW_E_ARG, "null output");
  if (!ws || ws_bytes < (size_t)kErrBytes) return fail(UW_E_WORKSPACE, "decode needs a %d-byte workspace", kErrBytes);
  DecArgs a;
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
  a.chunk = d->info.chunk;
  std::memset(a.pal, 0, 16);
  std::memcpy(a.pal, d->info.palette, 16);
  std::memcpy(a.len, d->info.code_len, 16);
  std::memcpy(a.code, d->info.code, 32);
  const dim3 grid((unsigned)d->info.tiles, (unsigned)std::max(1, (d->max_tile_chunks + 63) / 64));
  switch (mode) {
    case DEC_IDX: hipLaunchKernelGGL(k_decode<DEC_IDX>, grid, dim3(64), 0, s, a); break;
    case DEC_EXP: hipLaunchKernelGGL(k_decode<DEC_EXP>, grid, dim3(64), 0, s, a); break;
    default: hipLaunchKernelGGL(k_decode<DEC_BF16>, grid, dim3(64), 0, s, a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "decode launch: %s", hipGetErrorString(e));
  return UW_OK;
}

static void fill_gemm_args(const uw_dmat* d, GemmArgs& a, const uint16_t* x, float* y, int32_t m) {
  a.sm = d->sm;
  a.flags = d->flags;
  a.vprefix = d->vprefix;
  a.vexp = d->vexp;
  a.x = x;
  a.y = y;
  a.n = (int32_t)d->info.n;
  a.k = (int32_t)d->info.k;
  a.m = m;
  a.kb = (int32_t)d->info.kb;
  const uint32_t p0 = d->info.palette[0];
  a.base2 = (p0 << 7) | (p0 << 23);
  a.m0 = 0x000F000Fu;
  a.m1 = 0x00F000F0u;
  std::memcpy(a.tab, d->info.palette, 16);
}

}  // namespace uw

using namespace uw;

extern "C" {

size_t uw_dmat_size(void) { return sizeof(uw_dmat); }

uw_status uw_dmat_bind(uw_dmat* d, const void* blob_host, size_t bytes, const void* blob_dev, void* idx_dev) {
  if (!d || !blob_host || !blob_dev) return fail(UW_E_ARG, "null argument");
  uw_info info;
  uw_status st = validate_blob(blob_host, bytes, &info);
  if (st) return st;
  std::memset(d, 0, sizeof(*d));
  d->info = info;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(blob_dev);
  d->sm = base + info.sec_off[SEC_SM];
  d->flags = reinterpret_cast<const uint16_t*>(base + info.sec_off[SEC_FLAGS]);
  d->vprefix = reinterpret_cast<const uint32_t*>(base + info.sec_off[SEC_VPREFIX]);
  d->vexp = base + info.sec_off[SEC_VEXP];
  d->cbase = reinterpret_cast<const uint32_t*>(base + info.sec_off[SEC_CBASE]);
  d->off = reinterpret_cast<const uint32_t*>(base + info.sec_off[SEC_OFF]);
  d->words = reinterpret_cast<const uint32_t*>(base + info.sec_off[SEC_WORDS]);
  // Words readable without leaving the blob: the words section runs to the blob end, padded
  // to the section alignment when the caller copied the whole aligned blob.
  const uint64_t avail = (bytes > info.sec_off[SEC_WORDS] ? bytes - info.sec_off[SEC_WORDS] : 0) / 4;
  d->words_cap = (uint32_t)std::min<uint64_t>(avail, 0xFFFFFFFFull);
  d->idx = reinterpret_cast<uint8_t*>(idx_dev);
  const uint32_t* cb = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(blob_host) + info.sec_off[SEC_CBASE]);
  int32_t mx = 0;
  for (int64_t t = 0; t < info.tiles; ++t) mx = std::max<int32_t>(mx, (int32_t)(cb[t + 1] - cb[t]));
  d->max_tile_chunks = mx;
  const uint32_t* vp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(blob_host) + info.sec_off[SEC_VPREFIX]);
  int32_t mv = 0;
  for (int64_t t = 0; t < info.tiles; ++t) mv = std::max<int32_t>(mv, (int32_t)(vp[t + 1] - vp[t]));
  d->max_tile_verb = mv;
  d->magic = kDmatMagic;
  clear_error();
  return UW_OK;
}

uw_status uw_dmat_get_info(const uw_dmat* d, uw_info* out) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!out) return fail(UW_E_ARG, "null info");
  *out = d->info;
  clear_error();
  return UW_OK;
}

uw_status uw_workspace_size(const uw_dmat* d, int32_t m, int32_t op, size_t* bytes) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!bytes) return fail(UW_E_ARG, "null bytes");
  const uint64_t np = d->info.np, k = d->info.k, n = d->info.n;
  int32_t pipe = op;
  if (op == UW_PIPE_AUTO) {
    int32_t v;
    if (!autotune_lookup(n, k, m, &pipe, &v)) pipe = UW_PIPE_DIRECT_PALETTE;
  }
  switch (pipe) {
    case UW_PIPE_FULL_DECODE: *bytes = kErrBytes + align_up(2 * n * k, kAlign); break;
    case UW_PIPE_EXP_ONLY: *bytes = kErrBytes + align_up(np * k, kAlign); break;
    case UW_PIPE_TRANSCODE: *bytes = kErrBytes + align_up(np * k / 2, kAlign); break;
    case UW_PIPE_DIRECT_PALETTE: *bytes = 0; break;
    case UW_OP_DECODE_FULL:
    case UW_OP_TRANSCODE:
    case UW_OP_DECODE_EXP: *bytes = kErrBytes; break;
    default: return fail(UW_E_ARG, "unknown op %d", op);
  }
  clear_error();
  return UW_OK;
}

uw_status uw_decode_full(const uw_dmat* d, uint16_t* w_out, void* ws, size_t ws_bytes, hipStream_t s) {
  uw_status st = run_decode(d, DEC_BF16, reinterpret_cast<uint8_t*>(w_out), ws, ws_bytes, s);
  if (!st) clear_error();
  return st;
}

uw_status uw_transcode_palette(const uw_dmat* d, uint8_t* idx_out, void* ws, size_t ws_bytes, hipStream_t s) {
  uw_status st = run_decode(d, DEC_IDX, idx_out, ws, ws_bytes, s);
  if (!st) clear_error();
  return st;
}

uw_status uw_decode_exponents(const uw_dmat* d, uint8_t* exp_out, void* ws, size_t ws_bytes, hipStream_t s) {
  uw_status st = run_decode(d, DEC_EXP, exp_out, ws, ws_bytes, s);
  if (!st) clear_error();
  return st;
}

int32_t uw_variant_count(void) { return kNumVariants; }

const char* uw_variant_name(int32_t variant) {
  static char names[kNumVariants][48];
  if (variant < 0 || variant >= kNumVariants) return "";
  snprintf(names[variant], sizeof(names[variant]), "waves=%d unroll=%d", kVariants[variant].waves,
           kVariants[variant].unroll);
  return names[variant];
}

uw_status uw_gemm_variant(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t pipeline, int32_t variant,
                          void* ws, size_t ws_bytes, hipStream_t s) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!x || !y) return fail(UW_E_ARG, "null x or y");
  if (m < 1 || m > UW_MAX_M) return fail(UW_E_SHAPE, "m=%d outside [1, %d]", m, UW_MAX_M);
  if (variant < -1 || variant >= kNumVariants) return fail(UW_E_ARG, "bad variant %d", variant);
  if (pipeline == UW_PIPE_AUTO) {
    int32_t p, v;
    if (autotune_lookup(d->info.n, d->info.k, m, &p, &v)) {
      pipeline = p;
      if (variant < 0) variant = v;
    } else {
      pipeline = UW_PIPE_DIRECT_PALETTE;
    }
  }
  if (pipeline < UW_PIPE_FULL_DECODE || pipeline > UW_PIPE_DIRECT_PALETTE) return fail(UW_E_ARG, "bad pipeline %d", pipeline);
  if (variant < 0) variant = autotune_variant(d->info.n, d->info.k, m, pipeline);
  size_t need = 0;
  st = uw_workspace_size(d, m, pipeline, &need);
  if (st) return st;
  if (need && (!ws || ws_bytes < need)) return fail(UW_E_WORKSPACE, "pipeline %d needs %zu workspace bytes", pipeline, need);
  GemmArgs a;
  fill_gemm_args(d, a, x, y, m);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  const int pal_src = d->info.affine ? SRC_PAL_AFFINE : SRC_PAL_LUT;
  const int vs = d->max_tile_verb;
  switch (pipeline) {
    case UW_PIPE_DIRECT_PALETTE:
      if (!d->idx) return fail(UW_E_ARG, "direct palette needs an index stream bound at uw_dmat_bind");
      a.aux = d->idx;
      st = run_gemm(pal_src, a, d->info.tiles, variant, vs, s);
      break;
    case UW_PIPE_TRANSCODE:
      st = run_decode(d, DEC_IDX, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(pal_src, a, d->info.tiles, variant, vs, s);
      break;
    case UW_PIPE_EXP_ONLY:
      st = run_decode(d, DEC_EXP, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(SRC_EXP, a, d->info.tiles, variant, 0, s);
      break;
    default:
      st = run_decode(d, DEC_BF16, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(SRC_BF16, a, d->info.tiles, variant, 0, s);
      break;
  }
  if (!st) clear_error();
  return st;
}

uw_status uw_gemm(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t pipeline, void* ws, size_t ws_bytes,
                  hipStream_t s) {
  return uw_gemm_variant(d, x, y, m, pipeline, -1, ws, ws_bytes, s);
}

uw_status uw_gemm_bf16(const uint16_t* w, int64_t n, int64_t k, const uint16_t* x, float* y, int32_t m, int32_t variant,
                       hipStream_t s) {
  if (!w || !x || !y) return fail(UW_E_ARG, "null argument");
  if (n < 1 || k < 64 || n > (1 << 24)) return fail(UW_E_ARG, "bad shape");
  if (k % 64 || k > kMaxK) return fail(UW_E_SHAPE, "k=%lld must be a multiple of 64 up to %lld", (long long)k, (long long)kMaxK);
  if (m < 1 || m > UW_MAX_M) return fail(UW_E_SHAPE, "m=%d outside [1, %d]", m, UW_MAX_M);
  if (variant < -1 || variant >= kNumVariants) return fail(UW_E_ARG, "bad variant %d", variant);
  if (variant < 0) variant = autotune_variant(n, k, m, UW_PIPE_BF16);
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.aux = reinterpret_cast<const uint8_t*>(w);
  a.x = x;
  a.y = y;
  a.n = (int32_t)n;
  a.k = (int32_t)k;
  a.m = m;
  a.kb = (int32_t)(k / 64);
  uw_status st = run_gemm(SRC_BF16, a, (n + 15) / 16, variant, 0, s);
  if (!st) clear_error();
  return st;
}

uw_status uw_check(void* ws, hipStream_t s) {
  if (!ws) return fail(UW_E_ARG, "null workspace");
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(UW_E_HIP, "stream sync: %s", hipGetErrorString(e));
  uint32_t word = 0;
  e = hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(UW_E_HIP, "reading the error word: %s", hipGetErrorString(e));
  if (word) {
    const uint32_t zero = 0;
    e = hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(UW_E_HIP, "clearing the error word: %s", hipGetErrorString(e));
    return fail(UW_E_DATA, "a kernel found a corrupt stream (error word 0x%x)", word);
  }
  clear_error();
  return UW_OK;
}

uw_status uw_swiglu(const float* g, const float* u, uint16_t* h, int64_t count, hipStream_t s) {
  if (!g || !u || !h || count < 0) return fail(UW_E_ARG, "bad argument");
  if (count == 0) return UW_OK;
  const int64_t blocks = std::min<int64_t>((count + 255) / 256, 4096);
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, h, count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "swiglu launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

uw_status uw_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s) {
  if (!y || !x || m < 1 || n < 1) return fail(UW_E_ARG, "bad argument");
  hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)m), dim3(256), 0, s, y, x, n, eps);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "rmsnorm launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

}  // extern "C"
