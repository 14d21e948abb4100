// libuw device-facing C ABI (include/uw.h) for MI355X (gfx950): matrix views, workspace sizes,
// the decode and GEMM entry points (pipeline dispatch), the allocation-free GEMM, the error
// word, and the hard/easy MLP step scheduler.
//
// Method: Cloudflare blog post "Unweight": four-pipeline and autotuning paragraphs (the pipeline
// is chosen per matrix and batch size), hard/easy-layer paragraphs (the scheduler).
#include <cstdio>
#include <mutex>
#include <new>
#include <vector>

#include "uw_device.h"

using namespace uw;

namespace uw {
// The row decoder's lookup table for a matrix's code, built on the host and copied to the
// current device's table cache (uw_decode.hip).  Does nothing without a device.
void register_row_lut(const uw_info& info);
}  // namespace uw

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
  register_row_lut(info);
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

}  // extern "C"

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
  if (variant < -1 || variant >= uw_variant_count()) return fail(UW_E_ARG, "bad variant %d", variant);
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
  if (variant < -1 || variant >= uw_variant_count()) return fail(UW_E_ARG, "bad variant %d", variant);
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
  int decode_wgs = 0;        // decoder workgroups of a hard layer's decodes (0: the whole chip)
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
    const uw_status st = run_decode(d, DEC_IDX, d->idx, S->dws, S->dws_bytes, S->side, S->decode_wgs);
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

uw_status uw_sched_split(uw_sched* s, int32_t decode_workgroups) {
  if (!s || s->magic != uw::kSchedMagic || !s->impl) return fail(UW_E_ARG, "scheduler is not initialised");
  if (decode_workgroups < 0) return fail(UW_E_ARG, "decode_workgroups %d < 0", decode_workgroups);
  s->impl->decode_wgs = decode_workgroups;
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
