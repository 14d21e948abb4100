// Device-side definitions shared by libuw's HIP sources (uw_gemm.hip, uw_decode.hip,
// uw_glue.hip, uw_capi.hip): vector types, the bit-level rebuild helpers, buffer-resource loads
// and LDS-DMA, the GEMM and decoder argument blocks, and the host functions one source calls
// in another.  Not part of the public ABI.
//
// Method: Cloudflare blog post "Unweight".
//  - Reconstructive-matmul paragraphs: compressed weights are read from HBM, BF16 is rebuilt
//    on chip and fed straight to the matrix unit; the rebuilt matrix never reaches HBM.  Here
//    the rebuild happens in VGPRs, directly in the bf16 MFMA operand layout (CDNA MFMA reads
//    its operands from registers, unlike Hopper's shared-memory WGMMA operands).
//  - Rare-exponent paragraph: one decision per 64-weight segment; a verbatim segment swaps the
//    palette lookup for its raw exponent bytes.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <type_traits>

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

// =========================================================================================
// Reconstructive GEMM: operand source and argument block (kernels in uw_gemm.hip).
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

// Most K slices a multi-tile or wide-tile launch splits into (partial-sum planes).
constexpr int kMaxSlices = 16;

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

// Decoder output modes (kernels in uw_decode.hip).
enum DecMode { DEC_IDX = 0, DEC_EXP = 1, DEC_BF16 = 2 };

// =========================================================================================
// Host functions shared between the sources.
// =========================================================================================
inline uw_status check_dmat(const uw_dmat* d) {
  if (!d || d->magic != kDmatMagic) return fail(UW_E_ARG, "matrix view is not bound");
  return UW_OK;
}

inline void fill_gemm_args(const uw_dmat* d, GemmArgs& a, const uint16_t* x, float* y, int32_t m) {
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

// uw_gemm.hip: the GEMM launch (variant -1: the default for the shape), its K-slice plan, and
// the largest K-slice count any variant may take for a shape (workspace sizing).
uw_status run_gemm(int src, const GemmArgs& a, int64_t tiles, int variant, float* part, size_t part_bytes,
                   hipStream_t s);
int plan_gemm(int src, const GemmArgs& a, int64_t tiles, int* variant, const float* part, size_t part_bytes);
int64_t mt_max_slices(int64_t kb, int64_t tiles, int m);
// uw_decode.hip: Huffman decode of a bound matrix into `out` (mode DEC_*), error word in ws.
// max_wgs > 0: at most that many decoder workgroups (index and exponent output from chunks of
// at most 512 symbols; they take the units in turn), so the decode occupies only part of the
// chip; 0: as many as the units fill.
uw_status run_decode(const uw_dmat* d, int mode, uint8_t* out, void* ws, size_t ws_bytes, hipStream_t s,
                     int max_wgs = 0);
// uw_glue.hip: row-wise RMS norm of an fp32 [m, n] y into BF16 x.
bool rms_vec(const float* y, const uint16_t* x, int n);
hipError_t launch_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s);

}  // namespace uw
