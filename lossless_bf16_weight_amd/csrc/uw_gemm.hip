// libuw reconstructive GEMM for MI355X (gfx950): the per-tile, multi-tile and wide-tile
// kernels over palette, exponent and BF16 operand sources, the K-slice reductions, and their
// launchers (kernel variants, K-slice plans).
//
// Method: Cloudflare blog post "Unweight", reconstructive-matmul paragraphs (BF16 rebuilt on chip
// and fed to the matrix unit) and four-pipeline paragraphs (the consumers of pipelines 1-4).
#include <cstdio>

#include "uw_device.h"

namespace uw {

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
  // X rows, 1 KB (8 blocks of one row) a DMA; the launcher requires k % 512 == 0.  With an
  // unrolled ring whose waves each run blocks 0 .. kb-1 in order (shared X, or one wave a tile)
  // the rows are staged in parts of kXPart blocks: the first part here, the rest once the first
  // weights are out, each part checked by a barrier before its first block (see the ring), so
  // the start waits for 1/4 of X at k = 4096 instead of all of it.
  constexpr bool kXPartsOk = NB > 0 && XL;
  const bool xparts = kXPartsOk && (SHX || nw == 1);
  constexpr int kXPart = 16;
  const int per_row = a.k / 512;
  auto stage_x = [&](int cc0, int cc1) {  // chunks [cc0, cc1) of every valid row
    const int cpr = cc1 - cc0;
    for (int c = wave; c < mv * cpr; c += nw) {
      const int mr = c / cpr, cc = cc0 + (c - mr * cpr);
      lds_dma16(xrs, sx + (size_t)mr * xl_stride(a.k) + cc * 1024, (uint32_t)mr * a.k * 2 + cc * 1024 + lane * 16);
    }
  };
  if constexpr (XL) stage_x(0, xparts ? min(kXPart / 8, per_row) : per_row);
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
  if (xparts) stage_x(min(kXPart / 8, per_row), per_row);

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
      if constexpr (kXPartsOk) {
        if (xparts && i > 0 && i % kXPart == 0) {
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
  // Position of X row m's granules: rows of 256 bytes or more span all 64 banks, so 16
  // consecutive rows XOR their granule index with m & 15; 128-byte rows (one-block batches)
  // cover half the banks, so rows m and m + 8 would collide: there the XOR takes m >> 1.
  __host__ __device__ static constexpr int swz(int m) { return kGpr >= 16 ? (m & kSwz) : ((m >> 1) & kSwz); }
  static constexpr int kRows = 16 * CT;
  static constexpr int kBufBytes = kRows * kGpr * 16;     // one X batch
  static constexpr int kDmas = kRows * kGpr / 64;         // 1 KB LDS-DMA instructions per batch
};

// Rebuild the lane's 16 weights of one block as two bf16x8 MFMA operands.  fany: nonzero
// (wave-uniform) when some row the wave rebuilds has a verbatim segment in this block; f:
// the verbatim flags of the lane's own tile (bit r: its row).
template <int SRC, bool kNoBranch = false>
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
      if (kNoBranch || fany) {   // unbranched: the select keeps T where the lane's segment is coded
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
      const int q = (lane % C::kGpr) ^ C::swz(m);
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
  const int sw = C::swz(r);
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
  // The unrolled path's batch: the verbatim-exponent loads only when a block of the batch has a
  // verbatim row in this tile (a wave-uniform test; 92 % of an MLP matrix's tile-blocks have
  // none).  Issuing them costs the wave as much as any load, out of range or not.
  auto batch_has_verbatim = [&](int i) {
    uint32_t v = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) v |= __builtin_amdgcn_readlane(wfl, i * U + u);
    return v != 0u;
  };
  auto load_batch_nb = [&](int i, MtSlot<SRC>* sl) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_w(bs + i * U + u, sl[u]);
    if (kPal && batch_has_verbatim(i)) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_ev(bs + i * U + u, sl[u]);
    }
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
    if (NB == 0 || batch_has_verbatim(0)) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_ev(bs + u, sa[u]);
    }
  }
  if constexpr (NB > 0) {
    // Two batches deep.  Per batch a wave issues, in this order, its D X DMAs, 2U weight
    // loads and (palette sources, when the batch has a verbatim row) U verbatim-exponent
    // loads: at least LW loads after its DMAs.  Batch
    // i + 2 goes into the X buffer and register set of batch i - 1, which every wave finished
    // computing before the barrier of phase i.  Before that barrier a wave waits for its X DMAs
    // of batch i: loads retire in order and at that point batch i's weights (and batch i + 1's
    // DMAs and loads, once issued) follow them.  The count below leaves out the
    // verbatim-exponent loads, so it never exceeds the loads issued after the DMAs: the wait
    // covers them, and after a batch with verbatim loads it waits for a few loads more.  The
    // weights themselves are waited for by the compiler where compute reads them.
    constexpr int NBT = NB / U;
    constexpr int D = C::kDmas / R;
    constexpr int LW = 2 * U;
    if constexpr (NBT > 1) {
      issue_x(1, xb1);
      load_batch_nb(1, sl[1]);
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
        load_batch_nb(i + 2, sl[(i + 2) % 3]);
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
      const int q = (lane % C::kGpr) ^ C::swz(m);
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
      xoff[u][st] = (uint32_t)(xr * C::kGpr + ((u * 8 + 4 * h + st) ^ C::swz(xr))) * 16u;
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

// =========================================================================================
// Big-tile reconstructive GEMM for large batches (palette sources).
//
// The wide-tile kernel rebuilds a wave's weights for every 128-column X chunk, so at M in the
// hundreds the rebuild runs M/128 times over and its X reads from LDS feed only 32 weight
// rows.  Here a workgroup of 2 x NWM waves owns a BN x BM output tile (BN = 64 WN weight rows,
// BM = 64 WM X rows) and walks K one 64-column block at a time: the block's BN weight rows are
// rebuilt once, by the whole workgroup, into LDS as BF16, its BM X rows are staged by
// LDS-DMA, and each wave multiplies one (BN/2) x (BM/NWM) part with 32x32x16 MFMAs, both
// operands read from LDS (NWM = 4: two waves a SIMD, so one wave's issue stalls overlap the
// other's MFMAs).  Two blocks deep: while one block is multiplied, the next one's
// rebuilt weights and X rows are ready or landing and the one after is requested; one barrier
// a block.  LDS rows are 128 bytes (64 BF16), half the 64 banks; the 16-byte granule g of row
// r sits at position g ^ ((r >> 1) & 7), so any 16 consecutive rows' reads or writes of one
// granule hit 16 different 4-bank groups (rows r and r + 8 would share them under g ^ (r & 7)).
// Weight rows: wave w rebuilds tiles w*TW .. w*TW+TW-1 of the workgroup's BN/16, lane
// (r, g) the 16 weights it owns in the stored layout (row r, k = 16 g .. 16 g + 15) --
// the same loads and rebuild as the per-tile kernel, written out row-major.
// =========================================================================================
template <int SRC>
struct BigW {
  WRegs<SRC> w;
  u32x4 ev;
};

template <int SRC, int WN, int WM, int D, int NWM>
__global__ __launch_bounds__(128 * NWM) void k_gemm_big(GemmArgs a, float* part, int S) {
  static_assert(SRC <= SRC_PAL_LUT, "palette sources only");
  constexpr int BN = 64 * WN, BM = 64 * WM;
  constexpr int NW = 2 * NWM;                 // waves: 2 along the weight rows, NWM along X
  constexpr int CM = 2 * WM / NWM;            // 32-row X tiles a wave multiplies
  constexpr int TW = BN / 16 / NW;            // tiles a wave rebuilds
  constexpr int ABYTES = BN * 128, BBYTES = BM * 128;
  constexpr int XD = BBYTES / 1024 / NW;      // X DMAs (1 KB) a wave issues per block
  static_assert(TW >= 1 && TW * 16 * NW == BN && XD >= 1 && XD * 1024 * NW == BBYTES && CM * NWM == 2 * WM, "tile split");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (a.n + 15) >> 4;
  const int rg = blockIdx.x, s = blockIdx.y;
  const int mcol0 = blockIdx.z * BM;
  const int mv = min(BM, a.m - mcol0);
  const int bs = (int)((int64_t)s * a.kb / S), be = (int)((int64_t)(s + 1) * a.kb / S);
  const int nblk = be - bs;                   // <= 64: one block per lane in the flag registers

  // This wave's weight tiles t0w .. t0w + TW - 1 (nt of them inside the matrix) are
  // consecutive, so one buffer resource covers their sm streams, one their index streams and
  // one their verbatim exponents; per tile: stream offsets, flags of the slice (block bs + j
  // in lane j), and the verbatim rank of each block's first segment relative to the first
  // tile's verbatim base.
  const int t0w = rg * (BN / 16) + wave * TW;
  const int nt = max(0, min(TW, tiles - t0w));
  const size_t tb0 = nt ? (size_t)t0w * a.k * 16 : 0;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.sm + tb0, (uint32_t)nt * a.k * 16);
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(a.aux + tb0 / 2, (uint32_t)nt * a.k * 8);
  const uint32_t vbase = a.vprefix[nt ? t0w : 0];
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.vexp + (size_t)vbase * 64, (a.vprefix[nt ? t0w + nt : 0] - vbase) * 64);
  uint32_t so[TW], io[TW], wfl[TW], wvp[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int t = t0w + j;
    const bool ok = j < nt;
    so[j] = ok ? (uint32_t)(j * a.k * 16 + lane * 16) : kOob;
    io[j] = ok ? (uint32_t)(j * a.k * 8 + lane * 8) : kOob;
    const __amdgpu_buffer_rsrc_t frs = make_rsrc(a.flags + (ok ? (size_t)t * a.kb : 0), ok ? (uint32_t)a.kb * 2 : 0u);
    wfl[j] = __builtin_amdgcn_raw_buffer_load_b16(frs, lane < nblk ? (uint32_t)(bs + lane) * 2 : kOob, 0, 0);
    uint32_t before = 0;
    for (int c0 = 0; c0 < bs; c0 += 64) {
      const int b = c0 + lane;
      before += __popc((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(frs, b < bs ? (uint32_t)b * 2 : kOob, 0, 0));
    }
    before = wave_sum(before);
    const uint32_t v0 = ok ? a.vprefix[t] - vbase : 0u;
    uint32_t tot;
    wvp[j] = v0 + before + wave_excl_prefix_small<5>((uint32_t)__popc(wfl[j]), &tot);
  }

  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x + (size_t)mcol0 * a.k, (uint32_t)max(mv, 0) * a.k * 2);
  auto issue_x = [&](int b, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < XD; ++jj) {
      const int p = (wave * XD + jj) * 64 + lane;            // destination granule
      const int row = p >> 3, gs = (p & 7) ^ ((row >> 1) & 7);   // its source granule
      const uint32_t voff = (row < mv && b < be) ? (uint32_t)(row * a.k + b * 64 + gs * 8) * 2 : kOob;
      lds_dma16(xrs, buf + (wave * XD + jj) * 1024, voff);
    }
  };
  // Past the slice's last block the loads are issued all the same, out of range (zeros, no
  // traffic): every iteration issues the same NL instructions, so the compiler's and our
  // in-order vmcnt counts hold on every path.
  auto load_block = [&](int b, BigW<SRC> (&sl)[TW]) __attribute__((always_inline)) {
    const bool ok = b < be;
    const int jb = ok ? b - bs : 0;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      sl[j].w.s = bload16_nt(srs, ok ? so[j] : kOob, b * 1024);
      sl[j].w.i = bload8_nt(irs, ok ? io[j] : kOob, b * 512);
    }
    // Masks, not branches, inside: the multiply and rebuild of a block stay one basic block.
    // The verbatim-exponent loads go out only when one of the wave's tiles has a verbatim row
    // in the block (a wave-uniform test); the waits count none of them.
    const uint32_t okm = 0u - (uint32_t)ok;
    uint32_t fv = 0;
#pragma unroll
    for (int j = 0; j < TW; ++j) fv |= __builtin_amdgcn_readlane(wfl[j], jb) & okm;
    if (fv) {
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const uint32_t f = __builtin_amdgcn_readlane(wfl[j], jb) & okm;
        const uint32_t rank = __builtin_amdgcn_readlane(wvp[j], jb) + (uint32_t)__popc(f & ((1u << r) - 1u));
        const uint32_t vm = 0u - ((f >> r) & 1u);
        sl[j].ev = bload16(vrs, ((rank * 64 + g * 16) & vm) | (kOob & ~vm));
      }
    }
  };
  auto rebuild_to_lds = [&](int b, const BigW<SRC> (&sl)[TW], uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const uint32_t f = __builtin_amdgcn_readlane(wfl[j], b < be ? b - bs : 0) & (0u - (uint32_t)(b < be));
      u32x4 A0, A1;
      rebuild_block<SRC, true>(a, sl[j].w, f, f, r, sl[j].ev, A0, A1);
      const int row = (wave * TW + j) * 16 + r;
      *reinterpret_cast<u32x4*>(buf + row * 128 + (((2 * g) ^ ((row >> 1) & 7)) * 16)) = A0;
      *reinterpret_cast<u32x4*>(buf + row * 128 + (((2 * g + 1) ^ ((row >> 1) & 7)) * 16)) = A1;
    }
  };

  const int wn = wave / NWM, wm = wave % NWM;
  const int xr = lane & 31, hh = lane >> 5;
  floatx16 acc[WN][CM];
#pragma unroll
  for (int p = 0; p < WN; ++p)
#pragma unroll
    for (int c = 0; c < CM; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[p][c][e] = 0.f;
  // The operands of k-step st + 1 are read from LDS before the MFMAs of step st are issued.
  auto load_frags = [&](const uint8_t* A, const uint8_t* B, int st, u32x4 (&av)[WN], u32x4 (&bv)[CM]) __attribute__((always_inline)) {
    const int gr = 2 * st + hh;
#pragma unroll
    for (int p = 0; p < WN; ++p) {
      const int row = wn * 32 * WN + p * 32 + xr;
      av[p] = *reinterpret_cast<const u32x4*>(A + row * 128 + ((gr ^ ((row >> 1) & 7)) * 16));
    }
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      const int row = wm * 32 * CM + c * 32 + xr;
      bv[c] = *reinterpret_cast<const u32x4*>(B + row * 128 + ((gr ^ ((row >> 1) & 7)) * 16));
    }
  };
  auto compute = [&](const uint8_t* A, const uint8_t* B) __attribute__((always_inline)) {
    u32x4 av0[WN], bv0[CM], av1[WN], bv1[CM];
    load_frags(A, B, 0, av0, bv0);
    static_for<0, 4>([&](auto sc) __attribute__((always_inline)) {
      constexpr int st = decltype(sc)::value;
      u32x4 (&av)[WN] = (st & 1) ? av1 : av0;
      u32x4 (&bv)[CM] = (st & 1) ? bv1 : bv0;
      if constexpr (st + 1 < 4) {
        if constexpr (st & 1) load_frags(A, B, st + 1, av0, bv0);
        else load_frags(A, B, st + 1, av1, bv1);
      }
#pragma unroll
      for (int p = 0; p < WN; ++p)
#pragma unroll
        for (int c = 0; c < CM; ++c)
          acc[p][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[p]),
                                                              __builtin_bit_cast(bf16x8, bv[c]), acc[p][c], 0, 0, 0);
    });
  };
  // LDS-only barrier: each wave has already waited for its own loads and DMAs where needed.
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(63) & ~0x0F00);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Pipeline D blocks deep: block i is multiplied from A buffer i % 2 and X buffer
  // i % (D + 1) while the weights (registers) and X rows of blocks i + 1 .. i + D - 1 are in
  // flight or in place and block i + D's are requested; D register sets take blocks in turn
  // (the loop is unrolled by D for them).  A wave's loads of one block are NL instructions,
  // so before rebuilding block i + 1 it waits until at most the (D - 1) NL of the blocks after
  // it are outstanding (loads retire in order): that also covers its X DMAs of block i + 1,
  // which the barrier closing the step then publishes to the other waves.  Blocks past the
  // slice are loaded out of range (zeros, no traffic) and rebuilt into a buffer no one
  // multiplies.  One block's multiply and the next one's rebuild form one branch-free
  // region, which the scheduler is free to interleave.
  constexpr int NL = XD + 2 * TW;            // loads a wave issues per block, verbatim exponents aside
  static_assert(NL * (D - 1) <= 63, "vmcnt range");
  uint8_t* const abase = smem;
  uint8_t* const xbase = smem + 2 * ABYTES;
  auto abuf = [&](int j) __attribute__((always_inline)) { return abase + (j & 1) * ABYTES; };
  auto xbuf = [&](int j) __attribute__((always_inline)) { return xbase + (j % (D + 1)) * BBYTES; };
  BigW<SRC> sl[D][TW];
  // A block without verbatim rows loads no exponents and the rebuild's select masks them out:
  // start them defined.
#pragma unroll
  for (int jd = 0; jd < D; ++jd)
#pragma unroll
    for (int j = 0; j < TW; ++j) sl[jd][j].ev = u32x4{0, 0, 0, 0};
  static_for<0, D>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    issue_x(bs + j, xbuf(j));
    load_block(bs + j, sl[j]);
  });
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL * (D - 1)));
  rebuild_to_lds(bs, sl[0], abuf(0));
  barrier();
  // Step for block i (j = i mod D): request block i + D into the register set block i left,
  // multiply block i, rebuild block i + 1.
  auto step = [&](int i, auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    issue_x(bs + i + D, xbuf(i + D));
    load_block(bs + i + D, sl[j]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL * (D - 1)));
    compute(abuf(i), xbuf(i));
    rebuild_to_lds(bs + i + 1, sl[(j + 1) % D], abuf(i + 1));
    barrier();
  };
  // The loop's multiplies are unconditional (a conditional one would merge two versions of
  // the accumulators at the loop latch, which the compiler resolves by copying all of them
  // between register files every iteration); the last nblk % D blocks follow the loop.
  int i = 0;
  for (; i + D <= nblk; i += D) static_for<0, D>([&](auto jc) __attribute__((always_inline)) { step(i + decltype(jc)::value, jc); });
  static_for<0, D - 1>([&](auto jc) __attribute__((always_inline)) {
    if (i + decltype(jc)::value < nblk) step(i + decltype(jc)::value, jc);
  });
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));    // the out-of-range requests past the slice

  // D lane layout (32x32): X row (column of D) lane % 32 of column tile c; register e holds
  // weight row 8 (e / 4) + 4 hh + e % 4 of row pair p.  Unrolled at compile time (static_for):
  // an accumulator array indexed at run time would live in scratch memory.
  static_for<0, WN * CM * 4>([&](auto ic) __attribute__((always_inline)) {
    constexpr int p = decltype(ic)::value / (4 * CM), c = decltype(ic)::value / 4 % CM, qd = decltype(ic)::value % 4;
    const int mm = mcol0 + wm * 32 * CM + c * 32 + xr;
    const int n0 = rg * BN + wn * 32 * WN + p * 32 + 8 * qd + 4 * hh;
    if (mm >= a.m || n0 >= a.n) return;
    const floatx4 v{acc[p][c][4 * qd], acc[p][c][4 * qd + 1], acc[p][c][4 * qd + 2], acc[p][c][4 * qd + 3]};
    if (!part) {
      store_out4(a, mm, n0, v);
      return;
    }
    float* yp = part + (size_t)s * a.m * a.n + (size_t)mm * a.n + n0;
    if (n0 + 3 < a.n && (a.n & 3) == 0) {
      *reinterpret_cast<floatx4*>(yp) = v;
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (n0 + jj < a.n) yp[jj] = v[jj];
    }
  });
}

// y[i] = sum over s of part[s][i], in slice order.  A thread owns 4 consecutive elements
// and requests all S slices' values before adding them, so the loads overlap.
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

// =========================================================================================
// Host launchers
// =========================================================================================
// Kernel variants: kind 0 = per-tile kernel (waves split the tile's blocks; `unroll` blocks
// a batch), kind 1 = multi-tile kernel (`waves` row tiles a workgroup, X batches of `unroll`
// blocks in LDS, K split over workgroups), kind 2 = per-tile kernel with shared X (`waves`
// whole tiles a workgroup, all X rows in LDS once; M <= 16, k <= 4096, palette sources),
// kind 3 = wide-tile kernel (`waves` tile pairs a workgroup, 128 X rows a chunk, batches of
// `unroll` blocks; palette sources, other sources run the default multi-tile variant),
// kind 4 = big-tile kernel (64 * `waves` weight rows x 64 * `unroll` X rows a workgroup, W
// rebuilt once a block into LDS; palette sources, others run the default multi-tile variant);
// kind 5 = the big-tile kernel with the same tile split over eight waves (two a SIMD).
struct Variant {
  int kind;
  int waves;
  int unroll;
};
static const Variant kVariants[] = {{0, 4, 8}, {0, 2, 8}, {0, 8, 8},  {0, 16, 8}, {0, 1, 8}, {0, 4, 4}, {0, 2, 4},
                                    {0, 8, 4}, {0, 16, 4}, {0, 1, 4}, {1, 8, 4},  {1, 4, 4}, {1, 8, 2}, {1, 4, 2},
                                    {2, 2, 4}, {2, 4, 4}, {3, 4, 2}, {3, 8, 2}, {4, 2, 2}, {4, 2, 4}, {5, 2, 4}};
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
// Big-tile kernel: K slices so that the workgroups fill the chip once (one a compute unit at
// 128 KB of LDS, two at 80 KB), at most 64 blocks a slice.
// Big-tile pipeline depth and LDS bytes: two rebuilt-weight buffers and D + 1 X buffers of
// 64-element (128-byte) rows.  Three blocks in flight measured no faster than two at
// M = 128 .. 1024 on 14336 x 4096, so both tiles run two deep.
static constexpr int kBigDepth = 2;
static constexpr int big_lds(int WN, int WM, int D) { return 128 * (2 * 64 * WN + (D + 1) * 64 * WM); }
static int big_slices(int64_t tiles, int WN, int WM, int64_t kb, int m) {
  const int64_t wgs = ((tiles * 16 + 64 * WN - 1) / (64 * WN)) * ((m + 64 * WM - 1) / (64 * WM));
  const int64_t per_cu = big_lds(WN, WM, kBigDepth) <= 80 * 1024 ? 2 : 1;
  int64_t S = std::max<int64_t>(1, 256 * per_cu / std::max<int64_t>(wgs, 1));
  S = std::min<int64_t>(S, std::min<int64_t>(kb, kMaxSlices));
  return (int)std::max<int64_t>(S, (kb + 63) / 64);
}
// Upper bound of mt_slices, wide_slices and big_slices over the variants (groups * R >= tiles
// or tile pairs).
int64_t mt_max_slices(int64_t kb, int64_t tiles, int m) {
  int64_t S = std::max(slices_for(tiles * m_chunks(m), kb), slices_for((tiles + 1) / 2 * wide_chunks(m), kb));
  for (int v = 0; v < kNumVariants; ++v)
    if (kVariants[v].kind >= 4) S = std::max<int64_t>(S, big_slices(tiles, kVariants[v].waves, kVariants[v].unroll, kb, m));
  return S;
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
    if (U <= 2 && R == 8) return launch_mt_t<SRC, 8, 1, 8>(a, tiles, S, part, s);
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

template <int SRC, int WN, int WM, int D, int NWM>
static hipError_t launch_big_t(const GemmArgs& a, int64_t tiles, int S, float* part, hipStream_t s) {
  const dim3 grid((unsigned)((tiles * 16 + 64 * WN - 1) / (64 * WN)), (unsigned)S, (unsigned)((a.m + 64 * WM - 1) / (64 * WM)));
  hipLaunchKernelGGL((k_gemm_big<SRC, WN, WM, D, NWM>), grid, dim3(128 * NWM), big_lds(WN, WM, D), s, a, S > 1 ? part : nullptr, S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_reduce(a, S, part, s);
}

// 128 x 128 tiles (80 KB: two workgroups a CU) and 128 x 256 tiles (128 KB).  (256 x 256
// tiles need 256 accumulator registers a wave and run out of scalar registers for the stream
// descriptors.)
template <int SRC>
static hipError_t launch_big(const GemmArgs& a, int64_t tiles, int WM, bool eight, int S, float* part, hipStream_t s) {
  if (eight) return launch_big_t<SRC, 2, 4, kBigDepth, 4>(a, tiles, S, part, s);
  return WM == 4 ? launch_big_t<SRC, 2, 4, kBigDepth, 2>(a, tiles, S, part, s)
                 : launch_big_t<SRC, 2, 2, kBigDepth, 2>(a, tiles, S, part, s);
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
int plan_gemm(int src, const GemmArgs& a, int64_t tiles, int* variant, const float* part, size_t part_bytes) {
  const int ct = col_tiles(a.m);
  const bool pal = src <= SRC_PAL_LUT;
  if (*variant < 0) *variant = a.m > 16 ? kMtDefault : default_variant(tiles, a.kb, ct, a.m);
  if (kVariants[*variant].kind >= 3 && !pal) *variant = kMtDefault;
  const int kind = kVariants[*variant].kind;
  if (kind != 1 && kind != 3 && kind < 4) return 0;
  const int R = kVariants[*variant].waves;
  int S = kind >= 4 ? big_slices(tiles, R, kVariants[*variant].unroll, a.kb, a.m)
                    : kind == 3 ? wide_slices(tiles, R, a.kb, a.m) : mt_slices(tiles, R, a.kb, a.m);
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

uw_status run_gemm(int src, const GemmArgs& a, int64_t tiles, int variant, float* part,
                          size_t part_bytes, hipStream_t s) {
  int ct = col_tiles(a.m);
  const int S = plan_gemm(src, a, tiles, &variant, part, part_bytes);
  if (S > 0 && kVariants[variant].kind >= 4) {
    const int WM = kVariants[variant].unroll;
    const bool eight = kVariants[variant].kind == 5;
    const hipError_t e = src == SRC_PAL_AFFINE ? launch_big<SRC_PAL_AFFINE>(a, tiles, WM, eight, S, part, s)
                                               : launch_big<SRC_PAL_LUT>(a, tiles, WM, eight, S, part, s);
    if (e != hipSuccess) return fail(UW_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return UW_OK;
  }
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

}  // namespace uw

using namespace uw;

extern "C" {

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
  else if (kVariants[variant].kind == 4)
    snprintf(names[variant], sizeof(names[variant]), "big tile=%dx%d", 64 * kVariants[variant].waves,
             64 * kVariants[variant].unroll);
  else if (kVariants[variant].kind == 5)
    snprintf(names[variant], sizeof(names[variant]), "big tile=%dx%d waves=8", 64 * kVariants[variant].waves,
             64 * kVariants[variant].unroll);
  else
    snprintf(names[variant], sizeof(names[variant]), "multitile tiles=%d unroll=%d", kVariants[variant].waves,
             kVariants[variant].unroll);
  return names[variant];
}

}  // extern "C"
