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
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "uw_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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
// fp32 -> BF16, round to nearest even (finite inputs; the MLP glue's rounding).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
// SwiGLU of one element: bf16(silu(g) * u), silu(g) = g / (1 + e^-g).
__device__ __forceinline__ uint16_t swiglu1(float gv, float uv) { return f32_to_bf16(gv / (1.0f + expf(-gv)) * uv); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// (a & m) | (b & ~m) in one instruction (the compiler splits it into two for a literal mask).
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
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

// Exclusive prefix sum over the wave's lanes of a small per-lane value (< 2^BITS), and its
// total, by bit slices: each bit is balloted and the set lanes below this one counted (no LDS
// round trips, unlike shuffles).
template <int BITS>
__device__ __forceinline__ uint32_t wave_excl_prefix_small(uint32_t v, uint32_t* total) {
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int p = 0; p < BITS; ++p) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(((v >> p) & 1u) != 0u);
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << p;
    tot += (uint32_t)__popcll(m) << p;
  }
  *total = tot;
  return pre;
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
  float* y;                 // fp32 output, or unused with the SwiGLU epilogue
  const float* gate;        // SwiGLU epilogue: h = bf16(silu(gate) * y) replaces y (null: plain y)
  uint16_t* h;
  uint16_t* xn;             // K-slice reduction also writes xn = RMS-normed BF16 rows of y (null: no)
  float eps;
  int32_t n, k, m, kb;
  uint32_t base2;
  uint32_t tab[4];
  uint32_t m0, m1;  // 0x000F000F, 0x00F000F0 (see exps_affine)
};

// Final output of four consecutive elements of row mm, columns n0..n0+3 (those < n): fp32 Y,
// or with the SwiGLU epilogue h = bf16(silu(gate) * y) -- the same arithmetic as the separate
// SwiGLU kernel on the same y, so both routes give identical bits.
__device__ __forceinline__ void store_out4(const GemmArgs& a, int mm, int n0, floatx4 v) {
  const size_t o = (size_t)mm * a.n + n0;
  const bool full = n0 + 3 < a.n && (a.n & 3) == 0;
  if (a.gate) {
    if (full) {
      const floatx4 gv = *reinterpret_cast<const floatx4*>(a.gate + o);
      *reinterpret_cast<u32x2*>(a.h + o) = u32x2{(uint32_t)swiglu1(gv[0], v[0]) | ((uint32_t)swiglu1(gv[1], v[1]) << 16),
                                                 (uint32_t)swiglu1(gv[2], v[2]) | ((uint32_t)swiglu1(gv[3], v[3]) << 16)};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.n) a.h[o + j] = swiglu1(a.gate[o + j], v[j]);
    }
  } else {
    if (full) {
      *reinterpret_cast<floatx4*>(a.y + o) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.n) a.y[o + j] = v[j];
    }
  }
}

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
// also wait for every prefetched block behind it).  X rows (XL) can instead come from LDS.
// ev holds this lane's 16 raw exponents when its row's segment of the block is verbatim; the
// load is one unconditional instruction whose other lanes are out of range (no traffic).
template <int SRC, int CT, int XL>
struct Slot {
  WRegs<SRC> w;
  u32x4 xb0[XL ? 1 : CT], xb1[XL ? 1 : CT];  // B operand from global (zeros past the valid rows)
  u32x4 ev;                                   // palette sources: verbatim exponents
};

template <int CT, int U>
struct MaxThreads { static constexpr int v = CT == 1 ? (U >= 8 ? 512 : 1024) : (CT == 2 ? 512 : 256); };
static inline int max_waves(int ct, int unroll) { return ct == 1 ? (unroll >= 8 ? 8 : 16) : ct == 2 ? 8 : 4; }

__host__ __device__ constexpr int xl_stride(int k) { return 2 * k + 16; }  // padded X row in LDS
constexpr int kXlMaxBytes = 48 * 1024;

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1 (each index usable as
// a constant, e.g. in an s_waitcnt operand).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt operand that waits until at most n vector-memory loads are outstanding (lgkm and
// exp counters left alone): vmcnt bits 3:0 and 15:14.
__host__ __device__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Global -> LDS staging with LDS-DMA buffer loads (no VGPRs: the data goes straight to LDS;
// lane i of one instruction writes `size` bytes at lds + i*size).  Out-of-range lanes write
// zeros.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// LDS layout of k_gemm (bytes): X rows (XL, padded) | cross-wave partial sums (nw > 1).  The
// two do not overlap, so the epilogue needs a single barrier.
struct LdsLayout {
  uint32_t x, red, total;
};
__host__ __device__ inline LdsLayout lds_layout(int nw, int ct, bool xl, int mv, int k) {
  LdsLayout L;
  L.x = 0;
  L.red = xl ? (uint32_t)mv * xl_stride(k) : 0u;
  L.total = L.red + (nw > 1 ? (uint32_t)nw * ct * 64 * 16 : 0u);
  return L;
}

// NB > 0: every wave owns exactly NB blocks (the launcher checks kb == NB * waves) and the
// block loop is fully unrolled into a continuous prefetch ring: block i + U is requested just
// before block i is computed, so U blocks stay in flight and, with no registers carried
// around a loop, every wait covers exactly one block's loads.  NB == 0: batches of U blocks.
// SHX (shared X): each wave owns a whole tile of its own (tile blockIdx.x * waves + wave, all
// kb <= 64 blocks) instead of a K range of one tile; the workgroup's waves share one copy of
// the X rows in LDS and need no cross-wave sum.
template <int SRC, int CT, int U, int XL, int NB, int SHX>
__global__ __launch_bounds__((MaxThreads<CT, U>::v)) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int t = SHX ? (int)blockIdx.x * nw + wave : (int)blockIdx.x;
  const bool tile_ok = t * 16 < a.n;  // SHX: the last workgroup may hold tiles past n
  const int r = lane & 15, g = lane >> 4;
  const int kb = a.kb;
  const int b0 = SHX ? 0 : (int)((int64_t)wave * kb / nw), b1 = SHX ? kb : (int)((int64_t)(wave + 1) * kb / nw);
  const int nblk = b1 - b0;  // 1..64: the launcher keeps nw <= kb and every range within 64 blocks
  const int mcol0 = blockIdx.y * 16 * CT;
  const int mv = min(16 * CT, a.m - mcol0);  // valid X rows of this column block
  constexpr bool kPal = SRC <= SRC_PAL_LUT;
  const LdsLayout lay = lds_layout(SHX ? 1 : nw, CT, XL, mv, a.k);
  floatx4* red = reinterpret_cast<floatx4*>(smem + lay.red);
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
    const uint32_t tb = tile_ok ? (uint32_t)a.k * 16 : 0u;  // a tile past n reads zeros
    const size_t base = tile_ok ? tile_bytes : 0;
    wrs0 = make_rsrc(a.sm + base, tb);
    woff0 = lane * 16;
    if constexpr (SRC == SRC_EXP) {
      wrs1 = make_rsrc(a.aux + base, tb);
      woff1 = lane * 16;
    } else {
      wrs1 = make_rsrc(a.aux + base / 2, tb / 2);
      woff1 = lane * 8;
    }
  }
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (size_t)mcol0 * a.k, (uint32_t)mv * a.k * 2);
  uint32_t xoff[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) xoff[c] = 16 * c + r < mv ? (uint32_t)((16 * c + r) * a.k + g * 16) * 2 : kOob;
  // XL: LDS byte offset of this lane's X row.  Rows past mv read row 0: they only feed MFMA
  // output columns past mv, which are never stored.
  const uint32_t xl_off = (uint32_t)((r < mv ? r : 0) * xl_stride(a.k) + g * 32);

  // Verbatim bookkeeping (palette sources), all in registers: this wave's flags one block per
  // lane (wfl: bit r = row r's segment of the block is verbatim) and each block's rank among
  // the tile's verbatim segments (wvp: segments in earlier blocks of the tile).
  uint32_t wfl = 0, wvp = 0;
  __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vexp, 0);

  // Loads of block b; `ok` false turns every lane offset out of range (zeros, no traffic), so
  // a batch's loads are unconditional instructions even past the wave's last block.
  auto load_main = [&](int b, bool ok, Slot<SRC, CT, XL>& sl) {
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
  // This lane's verbatim exponents of block b (zeros unless its row's segment is verbatim).
  auto load_ev = [&](int b, bool ok, Slot<SRC, CT, XL>& sl) {
    if constexpr (kPal) {
      const int j = (b - b0) & 63;
      const uint32_t f = __builtin_amdgcn_readlane(wfl, j);
      const uint32_t rank = __builtin_amdgcn_readlane(wvp, j) + __popc(f & ((1u << r) - 1u));
      sl.ev = bload16(vrs, (ok && ((f >> r) & 1u)) ? rank * 64 + g * 16 : kOob);
    }
  };

  auto compute = [&](int b, const Slot<SRC, CT, XL>& sl) {
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
        const uint32_t f = __builtin_amdgcn_readlane(wfl, b - b0);
        if (f) {  // uniform: some row of this tile has a verbatim segment in block b
          const bool mine = (f >> r) & 1u;
          uint32_t R0[4], R1[4];
          exps_raw(sl.ev.x, sl.ev.y, R0);
          exps_raw(sl.ev.z, sl.ev.w, R1);
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
      if constexpr (XL) {  // X rows from LDS
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
  // Prologue, in issue order (loads retire in order, so each wait below covers only what it
  // needs): this wave's verbatim flags, the X rows (LDS-DMA), the first batch of weights --
  // nothing here waits on an earlier global load, so every wave's weight stream starts at
  // once -- then one barrier for the X rows, the verbatim prefix (bit-sliced ballots once the
  // flags are in) and the first batch's verbatim exponents.
  Slot<SRC, CT, XL> buf[NB > 0 ? NB : U];
  uint32_t fpre[4];
  __amdgpu_buffer_rsrc_t frs;
  if constexpr (kPal) {
    frs = make_rsrc(a.flags + (tile_ok ? (size_t)t * kb : 0), tile_ok ? (uint32_t)kb * 2 : 0u);
    wfl = __builtin_amdgcn_raw_buffer_load_b16(frs, lane < nblk ? (uint32_t)(b0 + lane) * 2 : kOob, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // flags of the tile's blocks before b0 (first 256)
      const int i = j * 64 + lane;
      fpre[j] = SHX ? 0u : __builtin_amdgcn_raw_buffer_load_b16(frs, i < b0 ? (uint32_t)i * 2 : kOob, 0, 0);
    }
  }
  // X rows, 1 KB (8 blocks of one row) a DMA; the launcher requires k % 512 == 0.  With shared
  // X and an unrolled ring the rows are staged in parts of kXPart blocks: the first part here,
  // the rest once the first weights are out, each part checked by a barrier before its first
  // block (see the ring), so the start waits for 1/4 of X at k = 4096 instead of all of it.
  constexpr bool kXParts = SHX && NB > 0 && XL;
  constexpr int kXPart = 16;
  const int per_row = a.k / 512;
  auto stage_x = [&](int cc0, int cc1) {  // chunks [cc0, cc1) of every valid row
    const int cpr = cc1 - cc0;
    for (int c = wave; c < mv * cpr; c += nw) {
      const int mr = c / cpr, cc = cc0 + (c - mr * cpr);
      lds_dma16(xrs, sx + (size_t)mr * xl_stride(a.k) + cc * 1024, (uint32_t)mr * a.k * 2 + cc * 1024 + lane * 16);
    }
  };
  if constexpr (XL) stage_x(0, kXParts ? min(kXPart / 8, per_row) : per_row);
#pragma unroll
  for (int u = 0; u < U; ++u) load_main(b0 + u, u < nblk, buf[u]);
  uint32_t vbase = 0, nvt = 0;
  if constexpr (kPal) {  // scalar loads (before the barrier, which would turn them into vector loads)
    const int tv = tile_ok ? t : 0;
    vbase = a.vprefix[tv];
    nvt = tile_ok ? a.vprefix[tv + 1] - vbase : 0u;
  }
  if constexpr (XL) {
    // This wave's X DMAs precede exactly the 2U weight loads above and loads retire in
    // order, so at most 2U outstanding means they have landed; then every wave's have.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * U));
    __syncthreads();
  }
  if constexpr (kPal) {
    vrs = make_rsrc(a.vexp + (size_t)vbase * 64, nvt * 64);
    uint32_t before = (uint32_t)__popc(fpre[0]) + __popc(fpre[1]) + __popc(fpre[2]) + __popc(fpre[3]);
    for (int j = 256; j < b0; j += 64) {  // tile rows of more than 256 + 64 blocks
      const int i = j + lane;
      before += __popc((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(frs, i < b0 ? (uint32_t)i * 2 : kOob, 0, 0));
    }
    uint32_t tot;
    wave_excl_prefix_small<9>(before, &tot);  // per lane at most 16 flags words of 16 bits
    wvp = tot + wave_excl_prefix_small<5>((uint32_t)__popc(wfl), &tot);
#pragma unroll
    for (int u = 0; u < U; ++u) load_ev(b0 + u, u < nblk, buf[u]);
  }
  if constexpr (kXParts) stage_x(min(kXPart / 8, per_row), per_row);

  if constexpr (NB > 0) {
    // A block's verbatim-exponent registers are read only when the block is flagged; the
    // allocator would reuse them as soon as an unflagged block is done, and overwriting the
    // destination of a load still in flight costs a wait for that load.  Each is kept alive
    // until block i + U is computed, by which point the in-order waits have retired it.
    auto keep = [](const u32x4& v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); };
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i + U < NB) {
        load_main(b0 + i + U, true, buf[i + U]);
        load_ev(b0 + i + U, true, buf[i + U]);
      }
      if constexpr (kPal)
        if (i >= U) keep(buf[i - U].ev);
      if constexpr (kXParts) {
        if (i > 0 && i % kXPart == 0) {
          // X part i / kXPart was requested before block i's weights, so once this wave has
          // waited for those (the empty asm use forces the wait here) its DMAs have landed;
          // the barrier then covers every wave's.
          if constexpr (SRC == SRC_BF16) keep(buf[i].w.w0); else keep(buf[i].w.s);
          __builtin_amdgcn_s_barrier();
        }
      }
      compute(b0 + i, buf[i]);
    }
    if constexpr (kPal) {
#pragma unroll
      for (int i = NB - U; i < NB; ++i) keep(buf[i].ev);
    }
  } else if constexpr (CT == 1 && XL && kPal) {
    // The same ring as a loop over U statically indexed slots: slot u holds block b + u and is
    // refilled with block b + u + U as soon as that block is computed.  Before the refill the
    // slot's exponent registers are held until their load has retired (it was issued right
    // after the block's weights, which compute just waited for).
    auto keep = [](const u32x4& v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); };
    for (int b = b0; b < b1; b += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u < b1) compute(b + u, buf[u]);
        keep(buf[u].ev);
        load_main(b + u + U, b + u + U < b1, buf[u]);
        load_ev(b + u + U, b + u + U < b1, buf[u]);
      }
    }
  } else {
    auto run_batch = [&](int b) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b + u < b1) compute(b + u, buf[u]);
    };
    run_batch(b0);
    for (int b = b0 + U; b < b1; b += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        load_main(b + u, b + u < b1, buf[u]);
        load_ev(b + u, b + u < b1, buf[u]);
      }
      run_batch(b);
    }
  }

#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] += acc2[c];
  // Epilogue: D lane layout = column m (lane%16), rows 4*(lane/16) + j.
  auto store = [&](int c, int l, floatx4 v) {
    const int mm = mcol0 + 16 * c + (l & 15);
    if (mm < a.m) store_out4(a, mm, t * 16 + 4 * (l >> 4), v);
  };
  if (nw == 1 || SHX) {
    if (tile_ok) {
#pragma unroll
      for (int c = 0; c < CT; ++c) store(c, lane, acc[c]);
    }
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
// Reconstructive GEMM for wider batches (multi-tile kernel).
//
// At M > 16 the per-tile kernel above re-reads the X columns for every 16-row tile, so X
// traffic from L2 grows with M x (n / 16) and dominates.  Here one workgroup of R waves
// holds R row tiles (one per wave) and a K-slice of the blocks; X is staged once per
// workgroup in LDS, in batches of U blocks (double-buffered LDS-DMA, no VGPRs), and every
// wave multiplies its rebuilt tile against it.  The K-slices of a row group (grid.y) write
// partial sums to the workspace when there are several, and a reduction kernel adds them
// in slice order (deterministic).
// LDS X batch: row m of 16*CT, U*8 granules of 16 bytes (8 bf16), granule q stored at
// position q ^ (m & 15 & (U*8-1)) of its row, so the 16 rows a B-operand load touches fall
// in distinct bank groups.
// =========================================================================================
template <int CT, int U>
struct MtCfg {
  static constexpr int kGpr = U * 8;                      // granules per X row of a batch
  static constexpr int kSwz = (kGpr - 1) < 15 ? (kGpr - 1) : 15;
  static constexpr int kRows = 16 * CT;
  static constexpr int kBufBytes = kRows * kGpr * 16;     // one X batch
  static constexpr int kDmas = kRows * kGpr / 64;         // 1 KB LDS-DMA instructions per batch
};

// Rebuild the lane's 16 weights of one block as two bf16x8 MFMA operands.  fany: nonzero
// (wave-uniform) when some row the wave rebuilds has a verbatim segment in this block; f:
// the verbatim flags of the lane's own tile (bit r: its row).
template <int SRC>
__device__ __forceinline__ void rebuild_block(const GemmArgs& a, const WRegs<SRC>& w, uint32_t fany, uint32_t f,
                                              int r, const u32x4& ev, u32x4& A0, u32x4& A1) {
  if constexpr (SRC == SRC_BF16) {
    A0 = w.w0;
    A1 = w.w1;
  } else {
    uint32_t T0[4], T1[4];
    if constexpr (SRC == SRC_PAL_AFFINE) {
      exps_affine(w.i.x, a.base2, a.m0, a.m1, T0);
      exps_affine(w.i.y, a.base2, a.m0, a.m1, T1);
    } else if constexpr (SRC == SRC_PAL_LUT) {
      exps_lut(w.i.x, a.tab, T0);
      exps_lut(w.i.y, a.tab, T1);
    } else {
      exps_raw(w.e.x, w.e.y, T0);
      exps_raw(w.e.z, w.e.w, T1);
    }
    if constexpr (SRC <= SRC_PAL_LUT) {
      if (fany) {
        uint32_t R0[4], R1[4];
        exps_raw(ev.x, ev.y, R0);
        exps_raw(ev.z, ev.w, R1);
        const uint32_t keep = ((f >> r) & 1u) ? 0u : ~0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          T0[j] = (T0[j] & keep) | (R0[j] & ~keep);
          T1[j] = (T1[j] & keep) | (R1[j] & ~keep);
        }
      }
    }
    uint32_t P0[4], P1[4];
    spread_sm(w.s.x, w.s.y, P0);
    spread_sm(w.s.z, w.s.w, P1);
    A0 = u32x4{(P0[0] & 0x807F807Fu) | T0[0], (P0[1] & 0x807F807Fu) | T0[1], (P0[2] & 0x807F807Fu) | T0[2],
               (P0[3] & 0x807F807Fu) | T0[3]};
    A1 = u32x4{(P1[0] & 0x807F807Fu) | T1[0], (P1[1] & 0x807F807Fu) | T1[1], (P1[2] & 0x807F807Fu) | T1[2],
               (P1[3] & 0x807F807Fu) | T1[3]};
  }
}

template <int SRC>
struct MtSlot {
  WRegs<SRC> w;
  u32x4 ev;
};

// part: S partial [m, n] fp32 planes (S > 1), or null to write y directly.
// NB > 0: every K slice holds exactly NB blocks (a multiple of U; the launcher checks), the
// batch loop is fully unrolled and runs two batches deep over three X buffers and three
// register sets (see the main loop); NB == 0: the loop below, one batch deep.
template <int SRC, int CT, int U, int R, int NB>
__global__ __launch_bounds__(64 * R) void k_gemm_mt(GemmArgs a, float* part, int S) {
  using C = MtCfg<CT, U>;
  static_assert(C::kDmas % R == 0, "every wave issues the same number of X DMAs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool kPal = SRC <= SRC_PAL_LUT;
  constexpr int kRowsPerDma = 64 / C::kGpr;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (a.n + 15) >> 4;
  const int t = blockIdx.x * R + wave;
  const bool tile_ok = t < tiles;
  const int s = blockIdx.y;
  const int bs = (int)((int64_t)s * a.kb / S), be = (int)((int64_t)(s + 1) * a.kb / S);
  const int nbatch = (be - bs + U - 1) / U;
  const int mcol0 = blockIdx.z * 16 * CT;
  const int mv = min(16 * CT, a.m - mcol0);

  // X batches: DMA j of a batch fills rows j*kRowsPerDma .. with granules permuted by row.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (size_t)mcol0 * a.k, (uint32_t)mv * a.k * 2);
  auto issue_x = [&](int batch, uint8_t* buf) {
    const int bb = bs + batch * U;
#pragma unroll
    for (int jj = 0; jj < C::kDmas / R; ++jj) {
      const int j = wave + jj * R;
      const int m = j * kRowsPerDma + lane / C::kGpr;
      const int q = (lane % C::kGpr) ^ (m & C::kSwz);
      const int blk = bb + (q >> 3);
      const uint32_t voff = (m < mv && blk < be) ? (uint32_t)(m * a.k + blk * 64 + (q & 7) * 8) * 2 : kOob;
      lds_dma16(xrs, buf + j * 1024, voff);
    }
  };

  // Weight streams of this wave's tile (bounds-checked; a missing tile reads zeros).
  const size_t tile_bytes = (size_t)t * a.k * 16;
  __amdgpu_buffer_rsrc_t wrs0, wrs1;
  uint32_t woff0 = kOob, woff1 = kOob;
  if constexpr (SRC == SRC_BF16) {
    const int rows = tile_ok ? min(16, a.n - t * 16) : 0;
    wrs0 = make_rsrc(a.aux + (tile_ok ? tile_bytes * 2 : 0), (uint32_t)rows * a.k * 2);
    wrs1 = wrs0;
    if (tile_ok && t * 16 + r < a.n) woff0 = (uint32_t)(r * a.k + g * 16) * 2;
  } else {
    wrs0 = make_rsrc(a.sm + (tile_ok ? tile_bytes : 0), tile_ok ? (uint32_t)a.k * 16 : 0u);
    if (tile_ok) woff0 = lane * 16;
    if constexpr (SRC == SRC_EXP) {
      wrs1 = make_rsrc(a.aux + (tile_ok ? tile_bytes : 0), tile_ok ? (uint32_t)a.k * 16 : 0u);
      if (tile_ok) woff1 = lane * 16;
    } else {
      wrs1 = make_rsrc(a.aux + (tile_ok ? tile_bytes / 2 : 0), tile_ok ? (uint32_t)a.k * 8 : 0u);
      if (tile_ok) woff1 = lane * 8;
    }
  }

  // Verbatim bookkeeping of this slice: flags of block bs + j in lane j (wfl), and each block's
  // rank among the tile's verbatim segments (wvp).  The flags are requested first; the ranks
  // are computed once they are in, after the first batch's weights have gone out.
  uint32_t wfl = 0, wvp = 0, fpre[4] = {0u, 0u, 0u, 0u};
  __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vexp, 0), frs = make_rsrc(a.flags, 0);
  if constexpr (kPal) {
    frs = make_rsrc(a.flags + (tile_ok ? (size_t)t * a.kb : 0), tile_ok ? (uint32_t)a.kb * 2 : 0u);
    wfl = __builtin_amdgcn_raw_buffer_load_b16(frs, lane < be - bs ? (uint32_t)(bs + lane) * 2 : kOob, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // flags of the tile's blocks before the slice (first 256)
      const int i = j * 64 + lane;
      fpre[j] = __builtin_amdgcn_raw_buffer_load_b16(frs, i < bs ? (uint32_t)i * 2 : kOob, 0, 0);
    }
  }

  auto load_w = [&](int b, MtSlot<SRC>& sl) {
    const bool ok = b < be;
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
  };
  auto load_ev = [&](int b, MtSlot<SRC>& sl) {
    if constexpr (kPal) {
      const bool ok = b < be;
      const int jb = ok ? b - bs : 0;
      const uint32_t f = __builtin_amdgcn_readlane(wfl, jb);
      const uint32_t rank = __builtin_amdgcn_readlane(wvp, jb) + (uint32_t)__popc(f & ((1u << r) - 1u));
      sl.ev = bload16(vrs, (ok && ((f >> r) & 1u)) ? rank * 64 + g * 16 : kOob);
    }
  };
  auto load_block = [&](int b, MtSlot<SRC>& sl) {
    load_w(b, sl);
    load_ev(b, sl);
  };

  constexpr bool kTwo = CT <= 2;   // a second accumulator set keeps back-to-back MFMAs independent
  floatx4 acc[CT], acc2[kTwo ? CT : 1];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < (kTwo ? CT : 1); ++c) acc2[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int sw = r & C::kSwz;
  // LDS byte offsets of this lane's X fragments in a batch (block u, MFMA step k2), column
  // tile 0: tile c adds the constant 16 * c * kGpr * 16 (the swizzle depends on r only).
  uint32_t xoff[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) xoff[u][k2] = (uint32_t)(r * C::kGpr + ((u * 8 + g * 2 + k2) ^ sw)) * 16u;

  auto load_batch = [&](int i, MtSlot<SRC>* sl) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_block(bs + i * U + u, sl[u]);
  };
  // X fragments of block u of the batch: column tile c, MFMA step k2 (x[c][0..1]).
  auto load_x = [&](const uint8_t* xbuf, int u, u32x4 (&x)[CT][2]) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      x[c][0] = *reinterpret_cast<const u32x4*>(xbuf + xoff[u][0] + c * 16 * C::kGpr * 16);
      x[c][1] = *reinterpret_cast<const u32x4*>(xbuf + xoff[u][1] + c * 16 * C::kGpr * 16);
    }
  };
  // One block: rebuild this lane's weights, then 2*CT MFMAs against the block's X fragments.
  auto mma_block = [&](int b, const MtSlot<SRC>& sl, const u32x4 (&x)[CT][2]) {
    uint32_t f = 0;
    if constexpr (kPal) f = __builtin_amdgcn_readlane(wfl, b - bs);
    u32x4 A0, A1;
    rebuild_block<SRC>(a, sl.w, f, f, r, sl.ev, A0, A1);
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, A0), a1 = __builtin_bit_cast(bf16x8, A1);
#pragma unroll
    for (int c = 0; c < CT; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, x[c][0]), acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if constexpr (kTwo)
        acc2[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, x[c][1]), acc2[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, x[c][1]), acc[c], 0, 0, 0);
    }
  };
  // A batch: the X fragments of block u+1 are read from LDS while block u is computed.
  auto compute_batch = [&](int i, const MtSlot<SRC>* sl, const uint8_t* xbuf) {
    const int b = bs + i * U;
    u32x4 xe[CT][2], xo[CT][2];
    load_x(xbuf, 0, xe);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b + u >= be) break;
      if (u + 1 < U) {
        if (u & 1) load_x(xbuf, u + 1, xe); else load_x(xbuf, u + 1, xo);
      }
      if (u & 1) mma_block(b + u, sl[u], xo); else mma_block(b + u, sl[u], xe);
    }
  };

  // Software pipeline, one batch deep: the weights and X of batch i+1 are requested before
  // batch i is computed, so they have a whole compute phase to arrive.  Two register sets
  // (sa, sb) and two X buffers alternate; each phase starts with a barrier after which
  // batch i's data is in place and batch i-1's X buffer is free.
  MtSlot<SRC> sl[NB > 0 ? 3 : 2][U];
  MtSlot<SRC>* const sa = sl[0];
  MtSlot<SRC>* const sb = sl[1];
  uint8_t* const xb1 = smem + C::kBufBytes;
  // Prologue in issue order: flags (above), X batch 0, the weights of batch 0, then the
  // tile's verbatim base (scalar), the ranks (bit-sliced ballots) and batch 0's verbatim
  // exponents -- no weight load waits on an earlier global load.
  issue_x(0, smem);
#pragma unroll
  for (int u = 0; u < U; ++u) load_w(bs + u, sa[u]);
  if constexpr (kPal) {
    const int tv = tile_ok ? t : 0;
    const uint32_t v0 = a.vprefix[tv];
    const uint32_t nv = tile_ok ? a.vprefix[tv + 1] - v0 : 0u;
    vrs = make_rsrc(a.vexp + (size_t)v0 * 64, nv * 64);
    uint32_t before = (uint32_t)__popc(fpre[0]) + __popc(fpre[1]) + __popc(fpre[2]) + __popc(fpre[3]);
    for (int j = 256; j < bs; j += 64) {  // tile rows of more than 256 + 64 blocks
      const int i = j + lane;
      before += __popc((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(frs, i < bs ? (uint32_t)i * 2 : kOob, 0, 0));
    }
    uint32_t tot;
    wave_excl_prefix_small<9>(before, &tot);
    wvp = tot + wave_excl_prefix_small<5>((uint32_t)__popc(wfl), &tot);
#pragma unroll
    for (int u = 0; u < U; ++u) load_ev(bs + u, sa[u]);
  }
  if constexpr (NB > 0) {
    // Two batches deep.  Per batch a wave issues, in this order, its D X DMAs, 2U weight
    // loads and (palette sources) U verbatim-exponent loads, LW loads after its DMAs.  Batch
    // i + 2 goes into the X buffer and register set of batch i - 1, which every wave finished
    // computing before the barrier of phase i.  Before that barrier a wave waits for its X DMAs
    // of batch i only: loads retire in order and at that point batch i's weights (and batch
    // i + 1's DMAs and loads, once issued) follow them, so the count below is exact; the
    // weights themselves are waited for by the compiler where compute reads them.
    constexpr int NBT = NB / U;
    constexpr int D = C::kDmas / R;
    constexpr int LW = 2 * U + (kPal ? U : 0);
    if constexpr (NBT > 1) {
      issue_x(1, xb1);
      load_batch(1, sl[1]);
    }
    static_for<0, NBT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      // Not __syncthreads(): its release fence would wait for every LDS-DMA in flight,
      // batch i + 1's included.  The explicit wait (this wave's batch-i DMAs; LDS reads of
      // batch i - 1 done) and a bare barrier suffice; the empty asm statements keep the
      // compiler from moving memory accesses across it.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(LW + (i + 1 < NBT ? D + LW : 0)) & ~0x0F00);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (i + 2 < NBT) {
        issue_x(i + 2, smem + ((i + 2) % 3) * C::kBufBytes);
        load_batch(i + 2, sl[(i + 2) % 3]);
      }
      compute_batch(i, sl[i % 3], smem + (i % 3) * C::kBufBytes);
    });
  } else {
  if constexpr (kPal) {
    // Batch 0 ready except, at most, its verbatim exponents (the last U loads; a flagged block
    // waits for its own when it reads them).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(U));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  for (int i = 0; i < nbatch; i += 2) {
    if (i > 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (i + 1 < nbatch) {
      load_batch(i + 1, sb);
      issue_x(i + 1, xb1);
    }
    compute_batch(i, sa, smem);
    if (i + 1 >= nbatch) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 2 < nbatch) {
      load_batch(i + 2, sa);
      issue_x(i + 2, smem);
    }
    compute_batch(i + 1, sb, xb1);
  }
  }
  if constexpr (kTwo) {
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] += acc2[c];
  }
  if (!tile_ok) return;
  // D lane layout: column lane % 16 of column tile c, rows 4 * (lane / 16) + j of the tile.
  const int n0 = t * 16 + 4 * g;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int mm = mcol0 + 16 * c + r;
    if (mm >= a.m) continue;
    if (!part) {  // one K slice: the final output
      store_out4(a, mm, n0, acc[c]);
      continue;
    }
    float* yp = part + (size_t)s * a.m * a.n + (size_t)mm * a.n + n0;
    if (n0 + 3 < a.n && (a.n & 3) == 0) {
      *reinterpret_cast<floatx4*>(yp) = acc[c];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < a.n) yp[j] = acc[c][j];
    }
  }
}

// =========================================================================================
// Wide-tile reconstructive GEMM for large batches (palette sources).
//
// At M in the hundreds the multi-tile kernel above is bound by LDS reads of X: every 16x32
// B fragment read feeds one 16-row tile.  Here a wave owns a pair of row tiles (32 rows) and
// uses 32x32x16 MFMAs, so one B fragment (32 X rows x 16 k) feeds 32 weight rows: half the
// LDS bytes and half the MFMA instructions per flop.  A workgroup of R waves holds R pairs
// and a chunk of 32*CW X rows (grid.z), staged per batch of U blocks in LDS exactly as in
// the multi-tile kernel; K slices (grid.y) write partial sums the same way.
// A fragments: lane l rebuilds row (l % 32) of the pair (tile (l / 16) % 2, row l % 16)
// for k = 32 h .. 32 h + 31 of each block (h = l / 32): the stored 16-weight groups of
// lanes r + 32 h and r + 32 h + 16 of its tile, rebuilt as in the other kernels.  MFMA step
// s (0..3) takes k = 32 h + 8 s .. + 7 from lane half h, so X granule 4 h + s.
// =========================================================================================
template <int SRC>
struct WideSlot {
  WRegs<SRC> wa, wb;
  u32x4 eva, evb;
};

template <int SRC, int CW, int U, int R>
__global__ __launch_bounds__(64 * R) void k_gemm_wide(GemmArgs a, float* part, int S) {
  static_assert(SRC <= SRC_PAL_LUT, "palette sources only");
  using C = MtCfg<2 * CW, U>;
  static_assert(C::kDmas % R == 0, "every wave issues the same number of X DMAs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int kRowsPerDma = 64 / C::kGpr;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, tsel = (lane >> 4) & 1, h = lane >> 5;
  const int tiles = (a.n + 15) >> 4;
  const int t0 = (blockIdx.x * R + wave) * 2;           // first tile of the wave's pair
  const int npt = max(0, min(2, tiles - t0));           // tiles of the pair (wave-uniform)
  const bool mine = tsel < npt;
  const int s = blockIdx.y;
  const int bs = (int)((int64_t)s * a.kb / S), be = (int)((int64_t)(s + 1) * a.kb / S);
  const int nbatch = (be - bs + U - 1) / U;
  const int mcol0 = blockIdx.z * 32 * CW;   // M chunks vary slowest: the row groups running
  const int mv = min(32 * CW, a.m - mcol0);   // together share one X chunk in L2

  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (size_t)mcol0 * a.k, (uint32_t)mv * a.k * 2);
  auto issue_x = [&](int batch, uint8_t* buf) {
    const int bb = bs + batch * U;
#pragma unroll
    for (int jj = 0; jj < C::kDmas / R; ++jj) {
      const int j = wave + jj * R;
      const int m = j * kRowsPerDma + lane / C::kGpr;
      const int q = (lane % C::kGpr) ^ (m & C::kSwz);
      const int blk = bb + (q >> 3);
      const uint32_t voff = (m < mv && blk < be) ? (uint32_t)(m * a.k + blk * 64 + (q & 7) * 8) * 2 : kOob;
      lds_dma16(xrs, buf + j * 1024, voff);
    }
  };

  // Both tiles of the pair behind one descriptor each (sign+mantissa, indices, flags).
  const size_t pair_sm = npt ? (size_t)t0 * a.k * 16 : 0;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.sm + pair_sm, (uint32_t)npt * a.k * 16);
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(a.aux + pair_sm / 2, (uint32_t)npt * a.k * 8);
  const uint32_t so = mine ? (uint32_t)(tsel * a.k * 16 + (r + 32 * h) * 16) : kOob;
  const uint32_t io = mine ? (uint32_t)(tsel * a.k * 8 + (r + 32 * h) * 8) : kOob;
  const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.flags + (npt ? (size_t)t0 * a.kb : 0), (uint32_t)npt * a.kb * 2);

  // Verbatim bookkeeping per tile i of the pair: flags of block bs + j in lane j (wfl[i]) and
  // each block's first rank among the pair's verbatim segments (wvp[i]).
  uint32_t wfl[2], wvp[2], fpre[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    wfl[i] = __builtin_amdgcn_raw_buffer_load_b16(frs, (i < npt && lane < be - bs) ? (uint32_t)(i * a.kb + bs + lane) * 2
                                                                                     : kOob, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = j * 64 + lane;
      fpre[i][j] = __builtin_amdgcn_raw_buffer_load_b16(frs, (i < npt && b < bs) ? (uint32_t)(i * a.kb + b) * 2 : kOob,
                                                        0, 0);
    }
  }
  auto load_w = [&](int b, WideSlot<SRC>& sl) {
    const bool ok = b < be;
    sl.wa.s = bload16_nt(srs, ok ? so : kOob, b * 1024);
    sl.wb.s = bload16_nt(srs, ok && so != kOob ? so + 256 : kOob, b * 1024);
    sl.wa.i = bload8_nt(irs, ok ? io : kOob, b * 512);
    sl.wb.i = bload8_nt(irs, ok && io != kOob ? io + 128 : kOob, b * 512);
  };
  __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vexp, 0);
  auto load_ev = [&](int b, WideSlot<SRC>& sl) {
    const bool ok = b < be;
    const int jb = ok ? b - bs : 0;
    const uint32_t f0 = __builtin_amdgcn_readlane(wfl[0], jb), f1 = __builtin_amdgcn_readlane(wfl[1], jb);
    const uint32_t p0 = __builtin_amdgcn_readlane(wvp[0], jb), p1 = __builtin_amdgcn_readlane(wvp[1], jb);
    const uint32_t f = tsel ? f1 : f0;
    const uint32_t rank = (tsel ? p1 : p0) + (uint32_t)__popc(f & ((1u << r) - 1u));
    const bool verb = ok && mine && ((f >> r) & 1u);
    sl.eva = bload16(vrs, verb ? rank * 64 + 32 * h : kOob);
    sl.evb = bload16(vrs, verb ? rank * 64 + 32 * h + 16 : kOob);
  };
  auto load_batch = [&](int i, WideSlot<SRC>* sl) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_w(bs + i * U + u, sl[u]);
      load_ev(bs + i * U + u, sl[u]);
    }
  };

  floatx16 acc[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  const int xr = lane & 31;                 // X row of the B fragment within a 32-row tile
  // LDS byte offsets of this lane's B fragments in a batch (block u, step st), column tile 0:
  // tile c adds the constant 32 * c * kGpr * 16 (the swizzle depends on xr only).
  uint32_t xoff[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      xoff[u][st] = (uint32_t)(xr * C::kGpr + ((u * 8 + 4 * h + st) ^ (xr & C::kSwz))) * 16u;
  // One block: rebuild the lane's 32 weights, then 4 * CW MFMAs (4 k-steps x CW column tiles).
  auto mma_block = [&](int b, int u, const WideSlot<SRC>& sl, const uint8_t* xbuf) {
    const uint32_t f0 = __builtin_amdgcn_readlane(wfl[0], b - bs), f1 = __builtin_amdgcn_readlane(wfl[1], b - bs);
    u32x4 A[4];
    rebuild_block<SRC>(a, sl.wa, f0 | f1, tsel ? f1 : f0, r, sl.eva, A[0], A[1]);
    rebuild_block<SRC>(a, sl.wb, f0 | f1, tsel ? f1 : f0, r, sl.evb, A[2], A[3]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, A[st]);
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xbuf + xoff[u][st] + c * 32 * C::kGpr * 16);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, xv), acc[c], 0, 0, 0);
      }
    }
  };
  auto compute_batch = [&](int i, const WideSlot<SRC>* sl, const uint8_t* xbuf) {
    const int b = bs + i * U;
    static_for<0, U>([&](auto uc) {   // u a compile-time constant: xoff stays in registers
      constexpr int u = decltype(uc)::value;
      if (b + u < be) mma_block(b + u, u, sl[u], xbuf);
    });
  };

  WideSlot<SRC> sa[U], sb[U];
  uint8_t* const xb1 = smem + C::kBufBytes;
  issue_x(0, smem);
#pragma unroll
  for (int u = 0; u < U; ++u) load_w(bs + u, sa[u]);
  {
    const int tv = npt ? t0 : 0;
    const uint32_t v0 = a.vprefix[tv];
    const uint32_t v1 = npt ? a.vprefix[tv + 1] : v0, v2 = npt ? a.vprefix[tv + npt] : v0;
    vrs = make_rsrc(a.vexp + (size_t)v0 * 64, (v2 - v0) * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t before = (uint32_t)__popc(fpre[i][0]) + __popc(fpre[i][1]) + __popc(fpre[i][2]) + __popc(fpre[i][3]);
      for (int j = 256; j < bs; j += 64) {  // tile rows of more than 256 + 64 blocks
        const int b = j + lane;
        before += __popc((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
            frs, (i < npt && b < bs) ? (uint32_t)(i * a.kb + b) * 2 : kOob, 0, 0));
      }
      uint32_t tot;
      wave_excl_prefix_small<9>(before, &tot);
      wvp[i] = (i ? v1 - v0 : 0u) + tot + wave_excl_prefix_small<5>((uint32_t)__popc(wfl[i]), &tot);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) load_ev(bs + u, sa[u]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < nbatch; i += 2) {
    if (i > 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (i + 1 < nbatch) {
      load_batch(i + 1, sb);
      issue_x(i + 1, xb1);
    }
    compute_batch(i, sa, smem);
    if (i + 1 >= nbatch) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 2 < nbatch) {
      load_batch(i + 2, sa);
      issue_x(i + 2, smem);
    }
    compute_batch(i + 1, sb, xb1);
  }
  if (!npt) return;
  // D lane layout (32x32): column lane % 32 of column tile c; register e holds pair row
  // 8 (e / 4) + 4 h + e % 4.
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const int mm = mcol0 + 32 * c + xr;
    if (mm >= a.m) continue;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int n0 = t0 * 16 + 8 * qd + 4 * h;
      if (n0 >= a.n) continue;
      const floatx4 v{acc[c][4 * qd], acc[c][4 * qd + 1], acc[c][4 * qd + 2], acc[c][4 * qd + 3]};
      if (!part) {
        store_out4(a, mm, n0, v);
        continue;
      }
      float* yp = part + (size_t)s * a.m * a.n + (size_t)mm * a.n + n0;
      if (n0 + 3 < a.n && (a.n & 3) == 0) {
        *reinterpret_cast<floatx4*>(yp) = v;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n0 + j < a.n) yp[j] = v[j];
      }
    }
  }
}

// y[i] = sum over s of part[s][i], in slice order.  A thread owns 4 consecutive elements
// and requests all S slices' values before adding them, so the loads overlap.
constexpr int kMaxSlices = 16;
// With gate set, the sum goes through the SwiGLU epilogue into h instead of y.
__global__ __launch_bounds__(256) void k_reduce_parts(const float* part, float* y, const float* gate, uint16_t* h,
                                                      int S, int64_t count) {
  const int64_t n4 = count >> 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    floatx4 v[kMaxSlices];
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s)
      if (s < S) v[s] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(part + (size_t)s * count) + i);
    floatx4 sum = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSlices; ++s)
      if (s < S) sum += v[s];
    if (gate) {
      const floatx4 gv = reinterpret_cast<const floatx4*>(gate)[i];
      reinterpret_cast<u32x2*>(h)[i] = u32x2{(uint32_t)swiglu1(gv[0], sum[0]) | ((uint32_t)swiglu1(gv[1], sum[1]) << 16),
                                             (uint32_t)swiglu1(gv[2], sum[2]) | ((uint32_t)swiglu1(gv[3], sum[3]) << 16)};
    } else {
      reinterpret_cast<floatx4*>(y)[i] = sum;
    }
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(size_t)s * count + i];
    if (gate)
      h[i] = swiglu1(gate[i], v);
    else
      y[i] = v;
  }
}

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
enum DecMode { DEC_IDX = 0, DEC_EXP = 1, DEC_BF16 = 2 };

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
// MLP glue (SwiGLU between up/gate and down; RMS norm feeding the next layer)
// =========================================================================================

__global__ void k_swiglu(const float* g, const float* u, uint16_t* h, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    h[i] = swiglu1(g[i], u[i]);
}

// Four elements a thread (count % 4 == 0, 16-byte aligned g and u, 8-byte aligned h).
__global__ void k_swiglu4(const floatx4* g, const floatx4* u, u32x2* h, int64_t count4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += (int64_t)gridDim.x * blockDim.x) {
    const floatx4 gv = g[i], uv = u[i];
    h[i] = u32x2{(uint32_t)swiglu1(gv[0], uv[0]) | ((uint32_t)swiglu1(gv[1], uv[1]) << 16),
                 (uint32_t)swiglu1(gv[2], uv[2]) | ((uint32_t)swiglu1(gv[3], uv[3]) << 16)};
  }
}

// Sum of squares of one float4 and the BF16 packing of a scaled float4, shared by the RMS-norm
// kernels so that every route computes the same bits.
__device__ __forceinline__ float rms_acc(float ss, floatx4 v) {
  return ss + (v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
}
__device__ __forceinline__ u32x2 rms_pack(floatx4 v, float scale) {
  return u32x2{(uint32_t)f32_to_bf16(v[0] * scale) | ((uint32_t)f32_to_bf16(v[1] * scale) << 16),
               (uint32_t)f32_to_bf16(v[2] * scale) | ((uint32_t)f32_to_bf16(v[3] * scale) << 16)};
}
__device__ __forceinline__ float rms_scale(float* part16, float ss, int n, float eps) {
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) part16[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += part16[w];
  return 1.0f / sqrtf(tot / (float)n + eps);
}

// K-slice reduction of the down projection with the RMS norm in it: one 1024-thread workgroup
// a row; each float4 of y is the in-order sum of its S slices (as k_reduce_parts), written to
// y, and the row is normalised as k_rmsnorm_v<V> does (same element grouping and order).
template <int V>
__global__ __launch_bounds__(1024) void k_reduce_rmsnorm(const float* part, float* y, uint16_t* xn, int S, int n,
                                                         int64_t count, float eps) {
  __shared__ float part16[16];
  const int n4 = n >> 2;
  const size_t row4 = (size_t)blockIdx.x * n4;
  floatx4 v[V];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    v[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (i < n4) {
      floatx4 p[kMaxSlices];
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q)
        if (q < S) p[q] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(part + (size_t)q * count) + row4 + i);
      v[j] = p[0];
#pragma unroll
      for (int q = 1; q < kMaxSlices; ++q)
        if (q < S) v[j] += p[q];
      reinterpret_cast<floatx4*>(y)[row4 + i] = v[j];
    }
    ss = rms_acc(ss, v[j]);
  }
  const float scale = rms_scale(part16, ss, n, eps);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    if (i < n4) reinterpret_cast<u32x2*>(xn)[row4 + i] = rms_pack(v[j], scale);
  }
}

// One 1024-thread workgroup a row, V float4 vectors a thread held in registers between the
// sum of squares and the scaling (n % 4 == 0, n <= 4096 * V).  Fixed reduction order: each
// thread's vectors in order, a butterfly inside each wave, then the 16 wave sums in order.
template <int V>
__global__ __launch_bounds__(1024) void k_rmsnorm_v(const float* y, uint16_t* x, int n, float eps) {
  __shared__ float part[16];   // wave sums
  const floatx4* yr = reinterpret_cast<const floatx4*>(y + (size_t)blockIdx.x * n);
  u32x2* xr = reinterpret_cast<u32x2*>(x + (size_t)blockIdx.x * n);
  const int n4 = n >> 2;
  floatx4 v[V];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    v[j] = i < n4 ? yr[i] : floatx4{0.f, 0.f, 0.f, 0.f};
    ss = rms_acc(ss, v[j]);
  }
  const float scale = rms_scale(part, ss, n, eps);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    if (i < n4) xr[i] = rms_pack(v[j], scale);
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
// Kernel variants: kind 0 = per-tile kernel (waves split the tile's blocks; `unroll` blocks
// a batch), kind 1 = multi-tile kernel (`waves` row tiles a workgroup, X batches of `unroll`
// blocks in LDS, K split over workgroups), kind 2 = per-tile kernel with shared X (`waves`
// whole tiles a workgroup, all X rows in LDS once; M <= 16, k <= 4096, palette sources),
// kind 3 = wide-tile kernel (`waves` tile pairs a workgroup, 128 X rows a chunk, batches of
// `unroll` blocks; palette sources, other sources run the default multi-tile variant).
struct Variant {
  int kind;
  int waves;
  int unroll;
};
static const Variant kVariants[] = {{0, 4, 8}, {0, 2, 8}, {0, 8, 8},  {0, 16, 8}, {0, 1, 8}, {0, 4, 4}, {0, 2, 4},
                                    {0, 8, 4}, {0, 16, 4}, {0, 1, 4}, {1, 8, 4},  {1, 4, 4}, {1, 8, 2}, {1, 4, 2},
                                    {2, 2, 4}, {2, 4, 4}, {3, 4, 2}, {3, 8, 2}};
static constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
static constexpr int kMtDefault = 10;   // {1, 8, 4}

static int col_tiles(int m) {
  const int ct = (m + 15) / 16;
  return ct <= 1 ? 1 : ct <= 2 ? 2 : ct <= 4 ? 4 : 8;
}

static int default_variant(int64_t tiles, int64_t kb, int ct, int m) {
  // Measured on MI355X: at M <= 4 one wave per tile with a 4-block ring is best on every MLP
  // shape (gate 14336 x 4096: 896 waves; down 4096 x 14336: 256 waves); otherwise about 2048
  // waves over the chip with 4-block batches; wider M keeps 4-block batches and fewer waves.
  const int cap = ct == 1 ? 16 : ct == 2 ? 8 : 4;
  const int64_t target = m <= 4 ? 128 : 1536;
  int w = 1;
  while (w < cap && tiles * w < target && kb / (w * 2) >= 4) w *= 2;
  for (int v = 0; v < kNumVariants; ++v)
    if (kVariants[v].kind == 0 && kVariants[v].waves == w && kVariants[v].unroll == 4) return v;
  return 0;
}

// Multi-tile kernel: K slices so that about 2048 waves run, each slice at most 64 blocks
// (one block per lane in the flag registers), at most kb slices.
// K slices of the multi-tile kernel: enough for about 2048 waves over the row groups and
// the M chunks of 16 * col_tiles(m) columns (grid.z), and at least one per 64 blocks (the
// palette kernels keep a slice's flags one block per lane).
static int64_t slices_for(int64_t waves_per_slice, int64_t kb) {
  int64_t S = (2048 + waves_per_slice - 1) / waves_per_slice;
  S = std::min<int64_t>(std::max<int64_t>(S, 1), std::min<int64_t>(kb, kMaxSlices));
  return std::max<int64_t>(S, (kb + 63) / 64);
}
static int64_t m_chunks(int m) { return (m + 16 * col_tiles(m) - 1) / (16 * col_tiles(m)); }
static int mt_slices(int64_t tiles, int R, int64_t kb, int m) {
  const int64_t groups = (tiles + R - 1) / R;
  return (int)slices_for(groups * R * m_chunks(m), kb);
}
constexpr int kWideCW = 4;   // 32-row X tiles per wide-tile workgroup (128 X rows a chunk)
static int64_t wide_chunks(int m) { return (m + 32 * kWideCW - 1) / (32 * kWideCW); }
static int wide_slices(int64_t tiles, int R, int64_t kb, int m) {
  const int64_t groups = ((tiles + 1) / 2 + R - 1) / R;
  return (int)slices_for(groups * R * wide_chunks(m), kb);
}
// Upper bound of mt_slices and wide_slices over the wave counts R (groups * R >= tiles or
// tile pairs).
static int64_t mt_max_slices(int64_t kb, int64_t tiles, int m) {
  return std::max(slices_for(tiles * m_chunks(m), kb), slices_for((tiles + 1) / 2 * wide_chunks(m), kb));
}

// Adds the S > 1 K-slice partial sums into y (or through the SwiGLU epilogue into h, or
// into y and the RMS-normed rows xn), in slice order.
static hipError_t launch_reduce(const GemmArgs& a, int S, float* part, hipStream_t s) {
  const int64_t count = (int64_t)a.m * a.n;
  if (a.xn) {  // the caller checked rms_fusable(): n % 4 == 0, n <= 16384, aligned y and xn
    const dim3 g((unsigned)a.m), b(1024);
    if (a.n <= 4096)
      hipLaunchKernelGGL((k_reduce_rmsnorm<1>), g, b, 0, s, part, a.y, a.xn, S, a.n, count, a.eps);
    else if (a.n <= 8192)
      hipLaunchKernelGGL((k_reduce_rmsnorm<2>), g, b, 0, s, part, a.y, a.xn, S, a.n, count, a.eps);
    else
      hipLaunchKernelGGL((k_reduce_rmsnorm<4>), g, b, 0, s, part, a.y, a.xn, S, a.n, count, a.eps);
    return hipGetLastError();
  }
  const int64_t blocks = std::min<int64_t>((count / 4 + 255) / 256 + 1, 4096);
  hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)blocks), dim3(256), 0, s, part, a.y, a.gate, a.h, S, count);
  return hipGetLastError();
}

template <int SRC, int CT, int U, int R>
static hipError_t launch_mt_t(const GemmArgs& a, int64_t tiles, int S, float* part, hipStream_t s) {
  using C = MtCfg<CT, U>;
  const dim3 grid((unsigned)((tiles + R - 1) / R), (unsigned)S, (unsigned)((a.m + 16 * CT - 1) / (16 * CT)));
  float* const pp = S > 1 ? part : nullptr;
  // Two batches deep (three X buffers) for the affine palette when every slice holds the same
  // block count of the MLP shapes (down_proj: 28 blocks at 8 slices; 8192^2: 32 at 4) and the
  // buffers stay within 64 KB, so several workgroups still share a CU.
  const int nbs = a.kb % S == 0 ? a.kb / S : 0;
  bool deep = false;
  if constexpr (SRC == SRC_PAL_AFFINE && 3 * C::kBufBytes <= 64 * 1024) {
    if (nbs % U == 0 && (nbs == 28 || nbs == 32)) {
      deep = true;
      if (nbs == 28)
        hipLaunchKernelGGL((k_gemm_mt<SRC, CT, U, R, 28>), grid, dim3(64 * R), 3 * C::kBufBytes, s, a, pp, S);
      else
        hipLaunchKernelGGL((k_gemm_mt<SRC, CT, U, R, 32>), grid, dim3(64 * R), 3 * C::kBufBytes, s, a, pp, S);
    }
  }
  if (!deep) hipLaunchKernelGGL((k_gemm_mt<SRC, CT, U, R, 0>), grid, dim3(64 * R), 2 * C::kBufBytes, s, a, pp, S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_reduce(a, S, part, s);
}

template <int SRC, int CT>
static hipError_t launch_mt_c(const GemmArgs& a, int64_t tiles, int R, int U, int S, float* part, hipStream_t s) {
  // Every wave issues the same number of X DMAs (2*CT*U a batch, a multiple of R); 128-row
  // batches use 2 blocks (64 KB of LDS, double-buffered).
  if constexpr (CT == 8) {
    return R == 8 ? launch_mt_t<SRC, 8, 2, 8>(a, tiles, S, part, s) : launch_mt_t<SRC, 8, 2, 4>(a, tiles, S, part, s);
  } else if constexpr (CT == 1) {
    return R == 8 ? launch_mt_t<SRC, 1, 4, 8>(a, tiles, S, part, s)
                  : (U >= 4 ? launch_mt_t<SRC, 1, 4, 4>(a, tiles, S, part, s) : launch_mt_t<SRC, 1, 2, 4>(a, tiles, S, part, s));
  } else {
    if (U >= 4)
      return R == 8 ? launch_mt_t<SRC, CT, 4, 8>(a, tiles, S, part, s) : launch_mt_t<SRC, CT, 4, 4>(a, tiles, S, part, s);
    return R == 8 ? launch_mt_t<SRC, CT, 2, 8>(a, tiles, S, part, s) : launch_mt_t<SRC, CT, 2, 4>(a, tiles, S, part, s);
  }
}

template <int SRC>
static hipError_t launch_mt(const GemmArgs& a, int64_t tiles, int R, int U, int S, float* part, hipStream_t s) {
  switch (col_tiles(std::min(a.m, 128))) {
    case 1: return launch_mt_c<SRC, 1>(a, tiles, R, U, S, part, s);
    case 2: return launch_mt_c<SRC, 2>(a, tiles, R, U, S, part, s);
    case 4: return launch_mt_c<SRC, 4>(a, tiles, R, U, S, part, s);
    default: return launch_mt_c<SRC, 8>(a, tiles, R, U, S, part, s);
  }
}

template <int SRC, int U, int R>
static hipError_t launch_wide_t(const GemmArgs& a, int64_t tiles, int S, float* part, hipStream_t s) {
  using C = MtCfg<2 * kWideCW, U>;
  const int64_t pairs = (tiles + 1) / 2;
  const dim3 grid((unsigned)((pairs + R - 1) / R), (unsigned)S, (unsigned)wide_chunks(a.m));
  hipLaunchKernelGGL((k_gemm_wide<SRC, kWideCW, U, R>), grid, dim3(64 * R), 2 * C::kBufBytes, s, a,
                     S > 1 ? part : nullptr, S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_reduce(a, S, part, s);
}

// Batches of 2 blocks only: 4 would spill at 8 waves a workgroup.
template <int SRC>
static hipError_t launch_wide(const GemmArgs& a, int64_t tiles, int R, int S, float* part, hipStream_t s) {
  return R == 8 ? launch_wide_t<SRC, 2, 8>(a, tiles, S, part, s) : launch_wide_t<SRC, 2, 4>(a, tiles, S, part, s);
}

struct Launch {
  int tiles, waves, unroll;
};

template <int SRC, int CT, int U, int XL, int NB, int SHX = 0>
static hipError_t launch_gemm_t(const GemmArgs& a, const Launch& L, hipStream_t s) {
  const int gy = (a.m + 16 * CT - 1) / (16 * CT);
  const size_t shm = lds_layout(SHX ? 1 : L.waves, CT, XL, std::min(a.m, 16 * CT), a.k).total;
  const unsigned gx = SHX ? (unsigned)((L.tiles + L.waves - 1) / L.waves) : (unsigned)L.tiles;
  hipLaunchKernelGGL((k_gemm<SRC, CT, U, XL, NB, SHX>), dim3(gx, gy), dim3(64 * L.waves), shm, s, a);
  return hipGetLastError();
}

// Shared-X launch: L.waves tiles a workgroup, each wave a whole tile row of kb blocks.
template <int SRC>
static hipError_t launch_gemm_shx(const GemmArgs& a, const Launch& L, hipStream_t s) {
  switch (a.kb) {
    case 16: return launch_gemm_t<SRC, 1, 4, 1, 16, 1>(a, L, s);
    case 32: return launch_gemm_t<SRC, 1, 4, 1, 32, 1>(a, L, s);
    case 64: return launch_gemm_t<SRC, 1, 4, 1, 64, 1>(a, L, s);
    default: return launch_gemm_t<SRC, 1, 4, 1, 0, 1>(a, L, s);
  }
}

// Fully unrolled ring (palette sources, X rows in LDS) for the per-wave block counts of the
// MLP shapes: k = 4096 over 2 or 4 waves, k = 14336 over 4 or 8 waves, k = 8192 over 2 waves.
template <int SRC, int U>
static hipError_t launch_gemm_ring(const GemmArgs& a, const Launch& L, hipStream_t s) {
  if (a.kb % L.waves == 0) {
    switch (a.kb / L.waves) {
      case 16: return launch_gemm_t<SRC, 1, U, 1, 16>(a, L, s);
      case 28: return launch_gemm_t<SRC, 1, U, 1, 28>(a, L, s);
      case 32: return launch_gemm_t<SRC, 1, U, 1, 32>(a, L, s);
      case 56: return launch_gemm_t<SRC, 1, U, 1, 56>(a, L, s);
      case 64: return launch_gemm_t<SRC, 1, U, 1, 64>(a, L, s);
      default: break;
    }
  }
  return launch_gemm_t<SRC, 1, U, 1, 0>(a, L, s);
}

template <int SRC, int CT, int XL>
static hipError_t launch_gemm_u(const GemmArgs& a, const Launch& L, hipStream_t s) {
  // Deeper prefetch only where the slot stays small enough to avoid spills (X from LDS).
  if constexpr (CT == 1 && XL && SRC <= SRC_PAL_LUT) {
    if (L.unroll >= 8) return launch_gemm_ring<SRC, 8>(a, L, s);
    return launch_gemm_ring<SRC, 4>(a, L, s);
  } else if constexpr (CT == 1) {
    if (L.unroll >= 8) return launch_gemm_t<SRC, 1, 8, XL, 0>(a, L, s);
    return launch_gemm_t<SRC, 1, 4, XL, 0>(a, L, s);
  } else {
    return launch_gemm_t<SRC, CT, 4, 0, 0>(a, L, s);
  }
}

template <int SRC, int CT>
static hipError_t launch_gemm_v(const GemmArgs& a, const Launch& L, hipStream_t s) {
  const int mv = std::min(a.m, 16);
  const bool xl = CT == 1 && a.k % 512 == 0 && (size_t)mv * xl_stride(a.k) <= (size_t)kXlMaxBytes;
  return xl ? launch_gemm_u<SRC, CT, CT == 1>(a, L, s) : launch_gemm_u<SRC, CT, 0>(a, L, s);
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

// part / part_bytes: workspace for the multi-tile kernel's K-slice partial sums (may be
// null: then it runs one slice, or the per-tile kernel when one slice cannot hold k).
// The kernel a GEMM call runs: resolves variant (-1: the default for the shape) and returns
// the multi-tile kernel's K-slice count, or 0 for the per-tile kernel (also when the
// multi-tile variant cannot run: not enough workspace for its slices).
static int plan_gemm(int src, const GemmArgs& a, int64_t tiles, int* variant, const float* part, size_t part_bytes) {
  const int ct = col_tiles(a.m);
  const bool pal = src <= SRC_PAL_LUT;
  if (*variant < 0) *variant = a.m > 16 ? kMtDefault : default_variant(tiles, a.kb, ct, a.m);
  if (kVariants[*variant].kind == 3 && !pal) *variant = kMtDefault;
  const int kind = kVariants[*variant].kind;
  if (kind != 1 && kind != 3) return 0;
  const int R = kVariants[*variant].waves;
  int S = kind == 3 ? wide_slices(tiles, R, a.kb, a.m) : mt_slices(tiles, R, a.kb, a.m);
  const size_t plane = (size_t)a.m * a.n * sizeof(float);
  if (S > 1 && (!part || part_bytes < (size_t)S * plane))
    S = part ? (int)std::min<size_t>(part_bytes / plane, (size_t)S) : 1;
  if (S < 1 || (pal && (a.kb + S - 1) / S > 64)) {
    *variant = default_variant(tiles, a.kb, ct, a.m);
    return 0;
  }
  return S;
}

// Largest dynamic LDS a workgroup may use on the current device (queried once per device).
static int lds_limit() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kXlMaxBytes;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
      v = kXlMaxBytes;
    cache[dev] = v;
  }
  return cache[dev];
}

static uw_status run_gemm(int src, const GemmArgs& a, int64_t tiles, int variant, float* part,
                          size_t part_bytes, hipStream_t s) {
  int ct = col_tiles(a.m);
  const int S = plan_gemm(src, a, tiles, &variant, part, part_bytes);
  if (S > 0 && kVariants[variant].kind == 3) {
    const int R = kVariants[variant].waves;
    const hipError_t e = src == SRC_PAL_AFFINE ? launch_wide<SRC_PAL_AFFINE>(a, tiles, R, S, part, s)
                                               : launch_wide<SRC_PAL_LUT>(a, tiles, R, S, part, s);
    if (e != hipSuccess) return fail(UW_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return UW_OK;
  }
  if (S > 0) {
    const int R = kVariants[variant].waves, U = kVariants[variant].unroll;
    hipError_t e;
    switch (src) {
      case SRC_PAL_AFFINE: e = launch_mt<SRC_PAL_AFFINE>(a, tiles, R, U, S, part, s); break;
      case SRC_PAL_LUT: e = launch_mt<SRC_PAL_LUT>(a, tiles, R, U, S, part, s); break;
      case SRC_EXP: e = launch_mt<SRC_EXP>(a, tiles, R, U, S, part, s); break;
      default: e = launch_mt<SRC_BF16>(a, tiles, R, U, S, part, s); break;
    }
    if (e != hipSuccess) return fail(UW_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return UW_OK;
  }
  Launch L;
  L.tiles = (int)tiles;
  L.unroll = kVariants[variant].unroll;
  if (kVariants[variant].kind == 2) {
    // Shared X needs the palette ring's conditions and every X row of the call in one
    // workgroup's LDS (up to the device's limit, so one such workgroup a CU at M = 16).
    const int mv = std::min(a.m, 16);
    const bool pal = src <= SRC_PAL_LUT;
    if (ct == 1 && pal && a.kb <= 64 && a.k % 512 == 0 && (size_t)mv * xl_stride(a.k) <= (size_t)lds_limit()) {
      L.waves = kVariants[variant].waves;
      const hipError_t e = src == SRC_PAL_AFFINE ? launch_gemm_shx<SRC_PAL_AFFINE>(a, L, s)
                                                 : launch_gemm_shx<SRC_PAL_LUT>(a, L, s);
      if (e != hipSuccess) return fail(UW_E_HIP, "gemm launch: %s", hipGetErrorString(e));
      return UW_OK;
    }
    variant = default_variant(tiles, a.kb, ct, a.m);
    L.unroll = kVariants[variant].unroll;
  }
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
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(blob_host);
  const uint32_t* cb = reinterpret_cast<const uint32_t*>(hb + info.sec_off[SEC_CBASE]);
  const uint32_t* of = reinterpret_cast<const uint32_t*>(hb + info.sec_off[SEC_OFF]);
  const uint16_t* fl = reinterpret_cast<const uint16_t*>(hb + info.sec_off[SEC_FLAGS]);
  // Decoder units: whole blocks whose chunks fill at most one wave, and the largest
  // bitstream slice any unit stages.
  d->dec_spc = info.chunk / kSeg;
  d->dec_cpb = (kTileRows + d->dec_spc - 1) / d->dec_spc;
  d->dec_nb = 64 / d->dec_cpb;
  uint32_t stage = 256;
  for (int64_t t = 0; t < info.tiles; ++t) {
    const int rows = (int)std::min<int64_t>(kTileRows, info.n - t * kTileRows);
    const uint32_t realmask = rows == kTileRows ? 0xFFFFu : ((1u << rows) - 1u);
    uint32_t c = cb[t];
    for (int64_t b0 = 0; b0 < info.kb; b0 += d->dec_nb) {
      uint32_t nch = 0;
      for (int64_t b = b0; b < std::min<int64_t>(b0 + d->dec_nb, info.kb); ++b)
        nch += ((uint32_t)__builtin_popcount(realmask & ~(uint32_t)fl[t * info.kb + b]) + d->dec_spc - 1) / d->dec_spc;
      if (nch) {
        const uint32_t wb = (of[c] >> 5) & ~3u, we = (of[c + nch] >> 5) + 3u;
        stage = std::max(stage, (we - wb + 255u) & ~255u);
      }
      c += nch;
    }
  }
  d->dec_stage_words = stage;
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
  const uint64_t parts = (uint64_t)mt_max_slices((int64_t)d->info.kb, (int64_t)d->info.tiles, std::max(m, 1)) *
                         (uint64_t)std::max(m, 1) * n * sizeof(float);
  switch (pipe) {
    case UW_PIPE_FULL_DECODE: *bytes = kErrBytes + align_up(2 * n * k, kAlign) + parts; break;
    case UW_PIPE_EXP_ONLY: *bytes = kErrBytes + align_up(np * k, kAlign) + parts; break;
    case UW_PIPE_TRANSCODE: *bytes = kErrBytes + align_up(np * k / 2, kAlign) + parts; break;
    case UW_PIPE_DIRECT_PALETTE: *bytes = kErrBytes + parts; break;
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
  if (kVariants[variant].kind == 0)
    snprintf(names[variant], sizeof(names[variant]), "waves=%d unroll=%d", kVariants[variant].waves,
             kVariants[variant].unroll);
  else if (kVariants[variant].kind == 2)
    snprintf(names[variant], sizeof(names[variant]), "shared-x tiles=%d unroll=%d", kVariants[variant].waves,
             kVariants[variant].unroll);
  else if (kVariants[variant].kind == 3)
    snprintf(names[variant], sizeof(names[variant]), "wide pairs=%d unroll=%d", kVariants[variant].waves,
             kVariants[variant].unroll);
  else
    snprintf(names[variant], sizeof(names[variant]), "multitile tiles=%d unroll=%d", kVariants[variant].waves,
             kVariants[variant].unroll);
  return names[variant];
}

}  // extern "C"

// Row-wise RMS norm of an fp32 [m, n] y into BF16 x (the vector kernel when the row fits it).
static bool rms_vec(const float* y, const uint16_t* x, int n) {
  return n % 4 == 0 && n <= 4 * 4096 && reinterpret_cast<uintptr_t>(y) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 8 == 0;
}
static hipError_t launch_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s) {
  const bool vec = rms_vec(y, x, n);
  if (vec && n <= 4096)
    hipLaunchKernelGGL((k_rmsnorm_v<1>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else if (vec && n <= 8192)
    hipLaunchKernelGGL((k_rmsnorm_v<2>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else if (vec)
    hipLaunchKernelGGL((k_rmsnorm_v<4>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)m), dim3(256), 0, s, y, x, n, eps);
  return hipGetLastError();
}

// Shared body of uw_gemm_variant, uw_gemm_swiglu and uw_gemm_rmsnorm: y (fp32); or
// h = bf16(silu(gate) * y) instead; or y and xn = RMS-normed rows of y.
static uw_status gemm_entry(const uw_dmat* d, const uint16_t* x, float* y, const float* gate, uint16_t* h, uint16_t* xn,
                            float eps, int32_t m, int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes,
                            hipStream_t s) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (!x || (gate ? !h : !y)) return fail(UW_E_ARG, gate ? "null x or h" : "null x or y");
  if (gate && ((reinterpret_cast<uintptr_t>(gate) & 15) || (reinterpret_cast<uintptr_t>(h) & 7)))
    return fail(UW_E_ARG, "gate must be 16-byte and h 8-byte aligned");
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
  // Workspace: [error word][decoded operand (pipelines 1-3)][K-slice partial sums].  The
  // decode pipelines need the first two; the partial sums are optional (without them the
  // multi-tile kernel runs one K slice or the per-tile kernel runs instead).
  const uint64_t np = d->info.np, k = d->info.k, n = d->info.n;
  uint64_t dec = 0;
  switch (pipeline) {
    case UW_PIPE_FULL_DECODE: dec = align_up(2 * n * k, kAlign); break;
    case UW_PIPE_EXP_ONLY: dec = align_up(np * k, kAlign); break;
    case UW_PIPE_TRANSCODE: dec = align_up(np * k / 2, kAlign); break;
    default: break;
  }
  if (dec && (!ws || ws_bytes < kErrBytes + dec))
    return fail(UW_E_WORKSPACE, "pipeline %d needs at least %llu workspace bytes", pipeline,
                (unsigned long long)(kErrBytes + dec));
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  float* part = nullptr;
  size_t part_bytes = 0;
  if (ws && ws_bytes > kErrBytes + dec) {
    part = reinterpret_cast<float*>(wsb + kErrBytes + dec);
    part_bytes = ws_bytes - kErrBytes - dec;
  }
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  fill_gemm_args(d, a, x, y, m);
  a.gate = gate;
  a.h = h;
  const int pal_src = d->info.affine ? SRC_PAL_AFFINE : SRC_PAL_LUT;
  // RMS norm: inside the K-slice reduction when the call runs one (same kernel choice as
  // run_gemm makes), else a separate pass over y after the GEMM.
  bool rms_fused = false;
  if (xn) {
    const int src = pipeline == UW_PIPE_EXP_ONLY ? SRC_EXP : pipeline == UW_PIPE_FULL_DECODE ? SRC_BF16 : pal_src;
    int v = variant;
    rms_fused = plan_gemm(src, a, d->info.tiles, &v, part, part_bytes) > 1 && rms_vec(y, xn, a.n);
    if (rms_fused) {
      a.xn = xn;
      a.eps = eps;
    }
  }
  switch (pipeline) {
    case UW_PIPE_DIRECT_PALETTE:
      if (!d->idx) return fail(UW_E_ARG, "direct palette needs an index stream bound at uw_dmat_bind");
      a.aux = d->idx;
      st = run_gemm(pal_src, a, d->info.tiles, variant, part, part_bytes, s);
      break;
    case UW_PIPE_TRANSCODE:
      st = run_decode(d, DEC_IDX, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(pal_src, a, d->info.tiles, variant, part, part_bytes, s);
      break;
    case UW_PIPE_EXP_ONLY:
      st = run_decode(d, DEC_EXP, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(SRC_EXP, a, d->info.tiles, variant, part, part_bytes, s);
      break;
    default:
      st = run_decode(d, DEC_BF16, wsb + kErrBytes, ws, ws_bytes, s);
      if (st) return st;
      a.aux = wsb + kErrBytes;
      st = run_gemm(SRC_BF16, a, d->info.tiles, variant, part, part_bytes, s);
      break;
  }
  if (!st && xn && !rms_fused) {
    const hipError_t e = launch_rmsnorm(y, xn, m, a.n, eps, s);
    if (e != hipSuccess) return fail(UW_E_HIP, "rmsnorm launch: %s", hipGetErrorString(e));
  }
  if (!st) clear_error();
  return st;
}

extern "C" {

uw_status uw_gemm_variant(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t pipeline, int32_t variant,
                          void* ws, size_t ws_bytes, hipStream_t s) {
  return gemm_entry(d, x, y, nullptr, nullptr, nullptr, 0.f, m, pipeline, variant, ws, ws_bytes, s);
}

uw_status uw_gemm(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t pipeline, void* ws, size_t ws_bytes,
                  hipStream_t s) {
  return gemm_entry(d, x, y, nullptr, nullptr, nullptr, 0.f, m, pipeline, -1, ws, ws_bytes, s);
}

uw_status uw_gemm_swiglu(const uw_dmat* d, const uint16_t* x, const float* gate, uint16_t* h, int32_t m,
                         int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!gate) return fail(UW_E_ARG, "null gate");
  return gemm_entry(d, x, nullptr, gate, h, nullptr, 0.f, m, pipeline, variant, ws, ws_bytes, s);
}

uw_status uw_gemm_rmsnorm(const uw_dmat* d, const uint16_t* x, float* y, uint16_t* xn, int32_t m, float eps,
                          int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!xn || !y) return fail(UW_E_ARG, "null y or xn");
  return gemm_entry(d, x, y, nullptr, nullptr, xn, eps, m, pipeline, variant, ws, ws_bytes, s);
}

}  // extern "C"

// =========================================================================================
// Allocation-free GEMM: the K-slice partial sums live in a device array of the library
// (kStaticScratchBytes a device, held until the process ends) instead of a caller workspace.
// Host code never passes the array's name to a kernel (in host code it is a stand-in, not a
// device address): its address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current.
// =========================================================================================
namespace uw {
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
}
static __device__ __align__(256) uint8_t scratch[uw::kErrBytes + uw::kStaticScratchBytes];

namespace uw {
static uw_status static_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(UW_E_HIP, "cannot query the current device");
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(UW_E_HIP, "device scratch of device %d: %s", dev, e != hipSuccess ? hipGetErrorString(e) : "null");
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return UW_OK;
}
}  // namespace uw

extern "C" {

uw_status uw_gemm_noalloc(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t variant, hipStream_t s) {
  uw_status st = check_dmat(d);
  if (st) return st;
  if (m < 1 || m > UW_MAX_M) return fail(UW_E_SHAPE, "m=%d outside [1, %d]", m, UW_MAX_M);
  size_t need = 0;
  if ((st = uw_workspace_size(d, m, UW_PIPE_DIRECT_PALETTE, &need))) return st;
  if (need - kErrBytes > kStaticScratchBytes)
    return fail(UW_E_WORKSPACE, "%lldx%lld at m=%d needs %zu bytes of K-slice partial sums; the allocation-free entry "
                "point holds %zu", (long long)d->info.n, (long long)d->info.k, m, need - kErrBytes, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws))) return st;
  return gemm_entry(d, x, y, nullptr, nullptr, nullptr, 0.f, m, UW_PIPE_DIRECT_PALETTE, variant, ws,
                    kErrBytes + kStaticScratchBytes, s);
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
  uw_status st = run_gemm(SRC_BF16, a, (n + 15) / 16, variant, nullptr, 0, s);
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
  const bool vec = count % 4 == 0 && reinterpret_cast<uintptr_t>(g) % 16 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(h) % 8 == 0;
  const int64_t items = vec ? count / 4 : count;
  const int64_t blocks = std::min<int64_t>((items + 255) / 256, 4096);
  if (vec)
    hipLaunchKernelGGL(k_swiglu4, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const floatx4*>(g),
                       reinterpret_cast<const floatx4*>(u), reinterpret_cast<u32x2*>(h), items);
  else
    hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, h, count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "swiglu launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

uw_status uw_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s) {
  if (!y || !x || m < 1 || n < 1) return fail(UW_E_ARG, "bad argument");
  const hipError_t e = launch_rmsnorm(y, x, m, n, eps, s);
  if (e != hipSuccess) return fail(UW_E_HIP, "rmsnorm launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

}  // extern "C"

// =========================================================================================
// Hard/easy scheduler (hard/easy-layer paragraphs of the post): hard layers keep only their
// bundle resident; their index streams are decoded on a side stream into one of two slot
// sets while the main stream computes the layers before them.
//   side:  [wait use_done[i%2]] decode hard layer i -> slot set i%2, record dec_done[i%2]
//   main:  ... [wait dec_done[i%2]] gate, up+SwiGLU, down+RMS norm of hard layer i,
//          record use_done[i%2], then enqueue the side work of hard layer i+2
// Two hard layers are decoded ahead at most; use_done is recorded once at set-up so that the
// first waits of every step (which cover the previous step's last uses) are always valid.
// =========================================================================================
namespace uw {
struct SchedImpl {
  int layers = 0, m = 0, hidden = 0, inter = 0;
  std::vector<uw_dmat> views;  // copies of the caller's views; hard ones index into a slot
  std::vector<uint8_t> hard;
  std::vector<int> hard_layers;  // layers with a hard matrix, in order
  size_t slot_bytes = 0;
  float* g = nullptr;
  uint16_t* h = nullptr;
  float* y = nullptr;
  uint16_t* xo = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* dws = nullptr;
  size_t dws_bytes = 0;
  float eps = 1e-5f;
  hipStream_t main = nullptr, side = nullptr;
  hipEvent_t dec_done[2] = {nullptr, nullptr}, use_done[2] = {nullptr, nullptr};
  uint8_t* trace = nullptr;  // per-layer copies of g, h, y and the layer output (uw_sched_trace)
};
// Bytes of one layer's record in a trace: g (fp32), h (BF16), y (fp32), layer output (BF16).
static size_t sched_trace_layer_bytes(const SchedImpl* S) {
  return (size_t)S->m * (6 * (size_t)S->inter + 6 * (size_t)S->hidden);
}
constexpr uint64_t kSchedMagic = 0x3130484353575555ull;  // "UUWSCH01"
}  // namespace uw

struct uw_sched {
  uint64_t magic;
  uw::SchedImpl* impl;
};

namespace uw {
static void sched_free_events(SchedImpl* S) {
  for (int i = 0; i < 2; ++i) {
    if (S->dec_done[i]) (void)hipEventDestroy(S->dec_done[i]);
    if (S->use_done[i]) (void)hipEventDestroy(S->use_done[i]);
    S->dec_done[i] = S->use_done[i] = nullptr;
  }
}

// Side-stream work of hard layer i: wait until the slot set's previous user is done, decode
// the layer's hard matrices into it, signal.
static uw_status sched_issue_decode(SchedImpl* S, int i) {
  const int set = i & 1, l = S->hard_layers[i];
  if (hipStreamWaitEvent(S->side, S->use_done[set], 0) != hipSuccess) return fail(UW_E_HIP, "stream wait failed");
  for (int j = 0; j < 3; ++j) {
    if (!S->hard[3 * l + j]) continue;
    const uw_dmat* d = &S->views[3 * l + j];
    const uw_status st = run_decode(d, DEC_IDX, d->idx, S->dws, S->dws_bytes, S->side);
    if (st) return st;
  }
  if (hipEventRecord(S->dec_done[set], S->side) != hipSuccess) return fail(UW_E_HIP, "event record failed");
  return UW_OK;
}
}  // namespace uw

extern "C" {

size_t uw_sched_size(void) { return sizeof(uw_sched); }

uw_status uw_sched_init(uw_sched* s, int32_t layers, int32_t m, int32_t hidden, int32_t inter,
                        const uw_dmat* const* mats, const uint8_t* hard, void* slots, size_t slot_bytes, float* g,
                        uint16_t* h, float* y, uint16_t* xo, void* ws, size_t ws_bytes, void* dws, size_t dws_bytes,
                        float eps, hipStream_t main_stream, hipStream_t side_stream) {
  if (!s || !mats || !hard || !g || !h || !y || !xo || !dws) return fail(UW_E_ARG, "null argument");
  s->magic = 0;
  s->impl = nullptr;
  if (layers < 1 || hidden < 1 || inter < 1) return fail(UW_E_ARG, "bad stack shape");
  if (m < 1 || m > UW_MAX_M) return fail(UW_E_SHAPE, "m=%d outside [1, %d]", m, UW_MAX_M);
  if ((reinterpret_cast<uintptr_t>(g) & 15) || (reinterpret_cast<uintptr_t>(h) & 7))
    return fail(UW_E_ARG, "g must be 16-byte and h 8-byte aligned");
  if (dws_bytes < (size_t)kErrBytes) return fail(UW_E_WORKSPACE, "the side error word needs %d bytes", kErrBytes);
  int n_hard = 0;
  for (int l = 0; l < layers; ++l) {
    for (int j = 0; j < 3; ++j) {
      const uw_dmat* d = mats[3 * l + j];
      uw_status st = check_dmat(d);
      if (st) return st;
      const int64_t en = j < 2 ? inter : hidden, ek = j < 2 ? hidden : inter;
      if (d->info.n != en || d->info.k != ek)
        return fail(UW_E_SHAPE, "layer %d matrix %d is %lldx%lld, expected %lldx%lld", l, j, (long long)d->info.n,
                    (long long)d->info.k, (long long)en, (long long)ek);
      if (hard[3 * l + j]) {
        ++n_hard;
        if (d->info.idx_bytes > slot_bytes)
          return fail(UW_E_WORKSPACE, "slot_bytes %zu < %llu index bytes of layer %d matrix %d", slot_bytes,
                      (unsigned long long)d->info.idx_bytes, l, j);
      } else if (!d->idx) {
        return fail(UW_E_ARG, "layer %d matrix %d is easy but has no index stream bound", l, j);
      }
    }
  }
  if (n_hard && !slots) return fail(UW_E_ARG, "hard matrices need slots");
  uw::SchedImpl* S = new (std::nothrow) uw::SchedImpl();
  if (!S) return fail(UW_E_NOMEM, "host allocation failed");
  S->layers = layers;
  S->m = m;
  S->hidden = hidden;
  S->inter = inter;
  S->views.resize(3 * (size_t)layers);
  S->hard.assign(hard, hard + 3 * (size_t)layers);
  for (int l = 0; l < layers; ++l) {
    bool any = false;
    for (int j = 0; j < 3; ++j) {
      S->views[3 * l + j] = *mats[3 * l + j];
      any = any || hard[3 * l + j];
    }
    if (any) {  // slot set by this hard layer's position among the hard layers
      const int set = (int)(S->hard_layers.size() & 1);
      for (int j = 0; j < 3; ++j)
        if (hard[3 * l + j])
          S->views[3 * l + j].idx = reinterpret_cast<uint8_t*>(slots) + ((size_t)set * 3 + j) * slot_bytes;
      S->hard_layers.push_back(l);
    }
  }
  S->slot_bytes = slot_bytes;
  S->g = g;
  S->h = h;
  S->y = y;
  S->xo = xo;
  S->ws = ws;
  S->ws_bytes = ws ? ws_bytes : 0;
  S->dws = dws;
  S->dws_bytes = dws_bytes;
  S->eps = eps;
  S->main = main_stream;
  S->side = side_stream;
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&S->dec_done[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&S->use_done[i], hipEventDisableTiming) != hipSuccess ||
        hipEventRecord(S->use_done[i], S->main) != hipSuccess) {
      uw::sched_free_events(S);
      delete S;
      return fail(UW_E_HIP, "event set-up failed");
    }
  }
  s->impl = S;
  s->magic = uw::kSchedMagic;
  clear_error();
  return UW_OK;
}

uw_status uw_sched_step(uw_sched* s, const uint16_t* x, uint16_t** out) {
  if (!s || s->magic != uw::kSchedMagic || !s->impl) return fail(UW_E_ARG, "scheduler is not initialised");
  if (!x || !out) return fail(UW_E_ARG, "null argument");
  uw::SchedImpl* S = s->impl;
  const int H = (int)S->hard_layers.size();
  uw_status st = UW_OK;
  for (int i = 0; i < std::min(H, 2) && !st; ++i) st = uw::sched_issue_decode(S, i);
  if (st) return st;
  const uint16_t* cur = x;
  int hi = 0;
  for (int l = 0; l < S->layers; ++l) {
    uint16_t* o = S->xo + (size_t)(l & 1) * S->m * S->hidden;
    const bool is_hard = hi < H && S->hard_layers[hi] == l;
    if (is_hard && hipStreamWaitEvent(S->main, S->dec_done[hi & 1], 0) != hipSuccess)
      return fail(UW_E_HIP, "stream wait failed");
    const uw_dmat* v = &S->views[3 * (size_t)l];
    st = gemm_entry(&v[0], cur, S->g, nullptr, nullptr, nullptr, 0.f, S->m, UW_PIPE_DIRECT_PALETTE, -1, S->ws,
                        S->ws_bytes, S->main);
    if (!st)
      st = gemm_entry(&v[1], cur, nullptr, S->g, S->h, nullptr, 0.f, S->m, UW_PIPE_DIRECT_PALETTE, -1, S->ws,
                          S->ws_bytes, S->main);
    if (!st)
      st = gemm_entry(&v[2], S->h, S->y, nullptr, nullptr, o, S->eps, S->m, UW_PIPE_DIRECT_PALETTE, -1, S->ws,
                          S->ws_bytes, S->main);
    if (st) return st;
    if (S->trace) {
      uint8_t* rec = S->trace + (size_t)l * uw::sched_trace_layer_bytes(S);
      const size_t gi = (size_t)S->m * S->inter, hd = (size_t)S->m * S->hidden;
      const void* src[4] = {S->g, S->h, S->y, o};
      const size_t len[4] = {4 * gi, 2 * gi, 4 * hd, 2 * hd};
      for (int q = 0; q < 4; ++q) {
        if (hipMemcpyAsync(rec, src[q], len[q], hipMemcpyDeviceToDevice, S->main) != hipSuccess)
          return fail(UW_E_HIP, "trace copy failed");
        rec += len[q];
      }
    }
    if (is_hard) {
      if (hipEventRecord(S->use_done[hi & 1], S->main) != hipSuccess) return fail(UW_E_HIP, "event record failed");
      if (hi + 2 < H && (st = uw::sched_issue_decode(S, hi + 2))) return st;
      ++hi;
    }
    cur = o;
  }
  *out = const_cast<uint16_t*>(cur);
  clear_error();
  return UW_OK;
}

uw_status uw_sched_trace(uw_sched* s, void* trace, size_t bytes) {
  if (!s || s->magic != uw::kSchedMagic || !s->impl) return fail(UW_E_ARG, "scheduler is not initialised");
  uw::SchedImpl* S = s->impl;
  const size_t need = (size_t)S->layers * uw::sched_trace_layer_bytes(S);
  if (trace && bytes < need) return fail(UW_E_WORKSPACE, "trace needs %zu bytes, got %zu", need, bytes);
  S->trace = reinterpret_cast<uint8_t*>(trace);
  clear_error();
  return UW_OK;
}

uw_status uw_sched_release(uw_sched* s) {
  if (!s || s->magic != uw::kSchedMagic || !s->impl) return fail(UW_E_ARG, "scheduler is not initialised");
  uw::sched_free_events(s->impl);
  delete s->impl;
  s->impl = nullptr;
  s->magic = 0;
  clear_error();
  return UW_OK;
}

}  // extern "C"
