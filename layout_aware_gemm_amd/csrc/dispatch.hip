// tgemm_run: validation, path selection, tile choice, workspace and launch.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <memory>
#include <mutex>
#include <vector>

#include "tgemm.h"
#include "tgemm_internal.h"

namespace tgemm {

// The no-allocation workspace of tgemm_run_noalloc: 64 MiB of device memory
// per device, held from the library's first use on that device until the
// process ends.  Host code never uses the array's name as an address: the
// device address of each device's copy comes from hipGetSymbolAddress,
// made once per device with that device current (scratch_address below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

int g_forced_tile = kTileAuto;
int g_forced_split = 0;
int g_fp8_cast_once = 1;  // tgemm_set_fp8_cast_once

inline bool is_n(char t) { return t == 'N' || t == 'n'; }

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// A dispatch packet's grid is at most 2^32 - 1 work-items.
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 24) - 1;

bool verbose() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("TGEMM_VERBOSE");
    v = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return v == 1;
}

// Tile choice.
//  - 256x256 tiles when they alone give most of the 256 compute units a
//    tile.
//  - Otherwise, for a store into C with both operands K-contiguous (NT)
//    and a long K, 256x256 tiles with K cut into `split` chunks so that
//    tiles x split fills the chip: a 256x256 tile moves half the operand
//    bytes per flop of a 128x128 one, which pays for writing and re-reading
//    the fp32 partials when every chunk still spans at least 2048 of K.
//  - Otherwise 128x128 tiles.
// Other splits are used only when requested.
int choose_tile(bool nt, int M, int N, int K, int epilogue, int* split) {
  const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
  const bool store = epilogue == TGEMM_EPI_STORE_BF16 || epilogue == TGEMM_EPI_STORE_F32;
  int cfg, s = 1;
  if (g_forced_tile != kTileAuto) {
    // (192x256 tiles exist for NT store epilogues only)
    cfg = g_forced_tile == kTile192 && !(nt && store) ? kTile256 : g_forced_tile;
  } else if (t256 >= 200) {
    cfg = kTile256;
  } else {
    const int64_t fill = 256 / t256, by_k = K / 2048;
    const int64_t auto_s = fill < by_k ? fill : by_k;
    // 192x256 tiles when M is a multiple of 192 and they keep as many
    // workgroups busy with fewer K chunks, so fewer fp32 partial products
    // (768x5120: 80 tiles x 3 chunks against 60 x 4)
    const int64_t t192 = (int64_t)ceil_div(M, 192) * ceil_div(N, 256);
    const int64_t f192 = 256 / t192, s192 = f192 < by_k ? f192 : by_k;
    if (nt && store && M % 192 == 0 && s192 >= 2 && t192 * s192 >= t256 * auto_s &&
        s192 < auto_s) {
      cfg = kTile192;
      s = (int)s192;
    } else if (nt && store && auto_s >= 2) {
      cfg = kTile256;
      s = (int)auto_s;
    } else {
      // A 128x128 tile does about 0.56x the work per compute unit of a
      // 256x256 one on NT, so 256x256 tiles win once they fill about half
      // the chip; the register-path layouts gain less from the big tile.
      // (Measured at K = 4096, 256 against 128 tiles: NT 4096x3072 96 vs
      // 131 us, 2048x4096 75 vs 78 us; NN / TN / TT at 144 tiles 129 / 159
      // / 146 vs 146 / 199 / 147 us, at 128 tiles 126 / 157 / 144 vs 89 /
      // 121 / 90 us.)
      cfg = t256 >= (nt ? 128 : 144) ? kTile256 : kTile128;
    }
  }
  if (g_forced_split > 0) s = g_forced_split;
  if (!store) s = 1;
  // every chunk holds at least one k-step
  const int max_s = ceil_div(K, 64);
  if (s > max_s) s = max_s;
  *split = s;
  return cfg;
}

int status_of(hipError_t e) { return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP; }

// ----------------------------------------------------------------------
// Workspace: the CE partials, the split-K partial products and the gemv
// partials.  Two sources.
//
// tgemm_run: one cached buffer per (device, stream).  Calls on one stream
// run in order, so each reuses the buffer the previous call on that stream
// used; growing it frees the old buffer and allocates the new one in
// stream order (hipFreeAsync / hipMallocAsync on that stream), so work
// still queued keeps a valid buffer.  A call holds the entry's lock from
// the lookup until its last kernel is enqueued, so two host threads that
// share a stream cannot grow (and free) a buffer the other has handed to
// kernels it has not yet enqueued.  Calls on different streams never share
// a buffer.  While the stream is being captured into a graph, a call gets a
// buffer of its own that is freed in stream order at its end (the graph
// owns it).  Cached buffers live until the process ends or until
// tgemm_release_workspace.
//
// tgemm_run_noalloc: the fixed device array `scratch` below, one per
// device, found once per device with hipGetSymbolAddress; no allocation.
// ----------------------------------------------------------------------
struct Workspace {
  void* ptr = nullptr;
  bool owned = false;                 // free in stream order at the end of this call
  std::unique_lock<std::mutex> hold;  // the cache entry, until the last launch is enqueued
};

struct WsEntry {
  int dev;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
  std::mutex mu;
};

std::mutex g_ws_mu;                               // guards the list itself
std::vector<std::unique_ptr<WsEntry>> g_ws;       // entries never move or go away

enum WsMode : int { kWsCached = 0, kWsScratch = 1 };

// (the array `scratch` is defined at file scope, below the anonymous
// namespace)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return TGEMM_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return TGEMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return TGEMM_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TGEMM_OK;
}

// Returns TGEMM_OK with w->ptr set, TGEMM_ERR_NO_MEMORY (allocation
// failed), TGEMM_ERR_WORKSPACE_LIMIT (scratch too small) or TGEMM_ERR_HIP.
int get_workspace(WsMode mode, hipStream_t s, size_t bytes, Workspace* w) {
  w->ptr = nullptr;
  w->owned = false;
  if (mode == kWsScratch) {
    if (bytes > kScratchBytes) return TGEMM_ERR_WORKSPACE_LIMIT;
    return scratch_address(&w->ptr);
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (s != nullptr && hipStreamIsCapturing(s, &cs) == hipSuccess &&
      cs != hipStreamCaptureStatusNone) {
    if (hipMallocAsync(&w->ptr, bytes, s) != hipSuccess || w->ptr == nullptr) {
      (void)hipGetLastError();
      return TGEMM_ERR_NO_MEMORY;
    }
    w->owned = true;
    return TGEMM_OK;
  }
  (void)hipGetLastError();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TGEMM_ERR_HIP;
  WsEntry* e = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    for (auto& x : g_ws)
      if (x->dev == dev && x->stream == s) e = x.get();
    if (e == nullptr) {
      g_ws.push_back(std::unique_ptr<WsEntry>(new WsEntry{dev, s, nullptr, 0, {}}));
      e = g_ws.back().get();
    }
  }
  w->hold = std::unique_lock<std::mutex>(e->mu);
  if (e->ptr != nullptr && e->bytes >= bytes) {
    w->ptr = e->ptr;
    return TGEMM_OK;
  }
  // grow by at least a quarter, so a slowly growing size does not
  // reallocate on every call
  size_t want = bytes;
  if (e->ptr != nullptr && want < e->bytes + e->bytes / 4) want = e->bytes + e->bytes / 4;
  void* p = nullptr;
  if (hipMallocAsync(&p, want, s) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    w->hold.unlock();
    return TGEMM_ERR_NO_MEMORY;
  }
  if (e->ptr != nullptr) (void)hipFreeAsync(e->ptr, s);
  e->ptr = p;
  e->bytes = want;
  w->ptr = p;
  return TGEMM_OK;
}

hipError_t release_workspace(Workspace& w, hipStream_t s) {
  const hipError_t e = w.owned ? hipFreeAsync(w.ptr, s) : hipSuccess;
  if (w.hold.owns_lock()) w.hold.unlock();
  return e;
}

hipError_t launch_gemm(char ta, char tb, int cfg, int epi, const GemmParams& p, hipStream_t s) {
  const bool an = is_n(ta), bn = is_n(tb);
  if (an && bn) return launch_gemm_nn(cfg, epi, p, s);
  if (an && !bn) return launch_gemm_nt(cfg, epi, p, s);
  if (!an && bn) return launch_gemm_tn(cfg, epi, p, s);
  return launch_gemm_tt(cfg, epi, p, s);
}

}  // namespace
}  // namespace tgemm

using namespace tgemm;

extern "C" int tgemm_set_split_k(int split) {
  if (split < 0 || split > 64) return TGEMM_ERR_INVALID_ARG;
  const int prev = g_forced_split;
  g_forced_split = split;
  return prev;
}

extern "C" int tgemm_set_fp8_cast_once(int enable) {
  if (enable != 0 && enable != 1) return TGEMM_ERR_INVALID_ARG;
  const int prev = g_fp8_cast_once;
  g_fp8_cast_once = enable;
  return prev;
}

extern "C" int tgemm_set_tile_config(int config) {
  if (config < kTileAuto || config > kTile192) return TGEMM_ERR_INVALID_ARG;
  const int prev = g_forced_tile;
  g_forced_tile = config;
  return prev;
}

extern "C" int tgemm_release_workspace(void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return TGEMM_ERR_HIP;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WsEntry* e = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    for (auto& x : g_ws)
      if (x->dev == dev && x->stream == s) e = x.get();
  }
  if (e == nullptr) return TGEMM_OK;
  std::lock_guard<std::mutex> hold(e->mu);
  hipError_t r = hipSuccess;
  if (e->ptr != nullptr) r = hipFreeAsync(e->ptr, s);
  e->ptr = nullptr;
  e->bytes = 0;
  return status_of(r);
}

namespace tgemm {
namespace {

// The whole of tgemm_run after validation, with the workspace taken from
// `mode`'s source.
int run_impl(WsMode mode, char transA, char transB, int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
             int epilogue, const int32_t* labels, float* out_loss, void* out_grad,
             hipStream_t s, float* out_scale = nullptr) {
  const int m = (int)M, n = (int)N, k = (int)K;

  // Element strides of the length-M / length-N vectors of a K=1 product.
  const int64_t sa = is_n(transA) ? lda : 1;
  const int64_t sb = is_n(transB) ? 1 : ldb;

  if (K == 1) {
    // Every K = 1 call runs pointwise, without matrix cores.
    hipError_t e;
    if (epilogue == TGEMM_EPI_CE) {
      if (verbose()) fprintf(stderr, "tgemm: K=1 pointwise cross-entropy\n");
      e = launch_k1_ce(static_cast<const uint16_t*>(A), sa, static_cast<const uint16_t*>(B), sb,
                       m, n, labels, out_loss, static_cast<uint16_t*>(out_grad), ldc, s);
      return status_of(e);
    }
    const int64_t groups = epilogue == TGEMM_EPI_ROPE_COSSIN ? (N + 7) / 8 : (N + 3) / 4;
    if ((M * groups + 255) / 256 > kMaxWorkgroups) return TGEMM_ERR_UNSUPPORTED;
    if (verbose()) fprintf(stderr, "tgemm: K=1 pointwise path, epilogue %d\n", epilogue);
    if (epilogue == TGEMM_EPI_ROPE_COSSIN)
      e = launch_k1_rope(static_cast<const int64_t*>(A), sa, static_cast<const float*>(B), sb, m,
                         n, static_cast<uint16_t*>(C), static_cast<uint16_t*>(out_grad), ldc, s);
    else if (epilogue == TGEMM_EPI_OUTER_F32)
      e = launch_k1_outer_f32(static_cast<const float*>(A), sa, static_cast<const float*>(B), sb,
                              m, n, static_cast<float*>(C), ldc, s);
    else
      e = launch_k1_outer_bf16(static_cast<const uint16_t*>(A), sa,
                               static_cast<const uint16_t*>(B), sb, m, n, C, ldc,
                               epilogue == TGEMM_EPI_STORE_F32, s);
    return status_of(e);
  }

  if ((M == 1 || N == 1) &&
      (epilogue == TGEMM_EPI_STORE_BF16 || epilogue == TGEMM_EPI_STORE_F32)) {
    // Matrix-vector or dot product: HBM-bound reductions, no matrix cores.
    const uint16_t* a = static_cast<const uint16_t*>(A);
    const uint16_t* b = static_cast<const uint16_t*>(B);
    int shape = kGemvRows;
    const uint16_t *X, *v;
    int64_t ldx = 0, sx = 1, sv, sc;
    int L;
    if (M == 1 && N == 1) {
      // dot product of op(A)[0, :] and op(B)[:, 0]; the unit-stride one is X
      const int64_t sa2 = is_n(transA) ? 1 : lda, sb2 = is_n(transB) ? ldb : 1;
      if (sa2 == 1 || sb2 != 1) {
        X = a, sx = sa2, v = b, sv = sb2;
      } else {
        X = b, sx = sb2, v = a, sv = sa2;
      }
      L = 1;
      sc = 1;
    } else if (N == 1) {
      // y[m] = op(A)[m, :] . op(B)[:, 0]
      v = b;
      sv = is_n(transB) ? ldb : 1;
      X = a;
      ldx = lda;
      shape = is_n(transA) ? kGemvRows : kGemvCols;
      L = m;
      sc = ldc;
    } else {
      // y[n] = op(A)[0, :] . op(B)[:, n]
      v = a;
      sv = is_n(transA) ? 1 : lda;
      X = b;
      ldx = ldb;
      shape = is_n(transB) ? kGemvCols : kGemvRows;
      L = n;
      sc = 1;
    }
    const int64_t nkc = gemv_chunks(shape, L, K);
    if (nkc * L > (int64_t(1) << 31)) return TGEMM_ERR_UNSUPPORTED;
    if (verbose())
      fprintf(stderr, "tgemm: %s M=%d N=%d K=%lld L=%d chunks=%lld\n",
              shape == kGemvRows ? "rowdot" : "colsweep", m, n, (long long)K, L, (long long)nkc);
    Workspace w;
    const int ws = get_workspace(mode, s, (size_t)(nkc * L) * sizeof(float), &w);
    if (ws != TGEMM_OK) return ws;
    hipError_t e = launch_gemv(shape, X, ldx, sx, v, sv, L, K, (int)nkc,
                               static_cast<float*>(w.ptr), C, sc,
                               epilogue == TGEMM_EPI_STORE_F32, s);
    const hipError_t ef = release_workspace(w, s);
    if (e == hipSuccess) e = ef;
    return status_of(e);
  }

  int split = 1;
  const int cfg = choose_tile(is_n(transA) && !is_n(transB), m, n, k, epilogue, &split);
  GemmParams p = {};
  p.A = static_cast<const uint16_t*>(A);
  p.B = static_cast<const uint16_t*>(B);
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = m;
  p.N = n;
  p.K = k;
  p.tilesM = ceil_div(M, tile_rows(cfg));
  p.tilesN = ceil_div(N, tile_cols(cfg));
  p.splitk = split;
  p.kchunk = split == 1 ? k : ceil_div(ceil_div(K, split), 64) * 64;
  if (split > 1) p.splitk = split = ceil_div(K, p.kchunk);  // no empty chunks
  if ((int64_t)p.tilesM * p.tilesN * p.splitk > kMaxWorkgroups) return TGEMM_ERR_UNSUPPORTED;
  p.groupM = p.tilesM < 4 ? p.tilesM : (p.tilesM <= 8 ? p.tilesM : 4);
  p.aligned = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0 &&
              lda % 8 == 0 && ldb % 8 == 0;
  if (verbose())
    fprintf(stderr,
            "tgemm: gemm %c%c M=%d N=%d K=%d tile=%d grid=%dx%d split=%d (chunk %d) groupM=%d "
            "aligned=%d epi=%d\n",
            transA, transB, m, n, k, cfg, p.tilesM, p.tilesN, p.splitk, p.kchunk, p.groupM,
            p.aligned, epilogue);

  if (epilogue != TGEMM_EPI_CE && split > 1) {
    // Split-K: one fp32 partial product per chunk (the fp32 store instance
    // writes it), then the sum in chunk order.
    const size_t ws_bytes = (size_t)split * (size_t)M * (size_t)N * sizeof(float);
    Workspace w;
    const int ws = get_workspace(mode, s, ws_bytes, &w);
    if (ws != TGEMM_OK) return ws;
    p.ws = static_cast<float*>(w.ptr);
    p.C = C;
    hipError_t e = launch_gemm(transA, transB, cfg, kEpiStoreF32, p, s);
    if (e == hipSuccess)
      e = launch_splitk_sum(p.ws, split, m, n, C, ldc, epilogue == TGEMM_EPI_STORE_F32, s);
    const hipError_t ef = release_workspace(w, s);
    if (e == hipSuccess) e = ef;
    return status_of(e);
  }

  if (epilogue != TGEMM_EPI_CE) {
    p.C = C;
    return status_of(launch_gemm(transA, transB, cfg,
                                 epilogue == TGEMM_EPI_STORE_BF16 ? kEpiStoreBf16 : kEpiStoreF32,
                                 p, s));
  }

  // Cross-entropy: GEMM + per-block partials, then the per-row combine,
  // then (with a gradient) the rescale pass -- or, for a deferred gradient
  // (out_scale set), the scale table the backward GEMMs apply on load.
  if (out_grad != nullptr && ((M * ((N + 7) / 8) + 255) / 256) > kMaxWorkgroups)
    return TGEMM_ERR_UNSUPPORTED;
  const int blk = ce_block_cols(cfg);
  const int nblk = p.tilesN * (tile_cols(cfg) / blk);
  const size_t ws_floats = 2 * (size_t)nblk * M + 2 * (size_t)M;
  Workspace w;
  const int ws = get_workspace(mode, s, ws_floats * sizeof(float), &w);
  if (ws != TGEMM_OK) return ws;
  float* wsf = static_cast<float*>(w.ptr);
  p.labels = labels;
  p.part_m = wsf;
  p.part_s = wsf + (size_t)nblk * M;
  p.ylabel = wsf + 2 * (size_t)nblk * M;
  float* lse = p.ylabel + M;
  p.grad = static_cast<uint16_t*>(out_grad);
  hipError_t e = launch_gemm(transA, transB, cfg, kEpiCE, p, s);
  if (e == hipSuccess)
    e = launch_ce_combine(p.part_m, p.part_s, p.ylabel, labels, m, n, nblk, out_loss, lse, s);
  if (e == hipSuccess && out_scale != nullptr)
    e = launch_ce_scale(p.part_m, lse, m, n, blk, out_scale, s);
  else if (e == hipSuccess && out_grad != nullptr)
    e = launch_ce_grad_fixup(p.grad, ldc, p.part_m, lse, labels, m, n, blk, s);
  const hipError_t ef = release_workspace(w, s);
  if (e == hipSuccess) e = ef;
  return status_of(e);
}

}  // namespace
}  // namespace tgemm

extern "C" int tgemm_run(char transA, char transB, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                         int64_t ldc, int epilogue, const int32_t* labels, float* out_loss,
                         void* out_grad, void* stream) {
  const int st = tgemm_validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, labels,
                                out_loss, out_grad);
  if (st != TGEMM_OK) return st;
  return run_impl(kWsCached, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, labels,
                  out_loss, out_grad, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int tgemm_run_noalloc(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                                 int64_t ldc, int epilogue, const int32_t* labels,
                                 float* out_loss, void* out_grad, void* stream) {
  const int st = tgemm_validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, labels,
                                out_loss, out_grad);
  if (st != TGEMM_OK) return st;
  return run_impl(kWsScratch, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, labels,
                  out_loss, out_grad, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int64_t tgemm_noalloc_scratch_bytes(void) { return (int64_t)kScratchBytes; }

extern "C" int tgemm_run_ce_deferred(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                     const void* A, int64_t lda, const void* B, int64_t ldb,
                                     const int32_t* labels, float* out_loss, void* out_e,
                                     int64_t lde, float* out_scale, void* stream) {
  if (out_e == nullptr || out_scale == nullptr) return TGEMM_ERR_INVALID_ARG;
  const int st = tgemm_validate(transA, transB, M, N, K, A, lda, B, ldb, nullptr, lde,
                                TGEMM_EPI_CE, labels, out_loss, out_e);
  if (st != TGEMM_OK) return st;
  // (a K = 1 product takes the pointwise path, which writes the finished
  // gradient; there is no deferred form of it)
  if (K == 1) return TGEMM_ERR_UNSUPPORTED;
  return run_impl(kWsCached, transA, transB, M, N, K, A, lda, B, ldb, nullptr, lde, TGEMM_EPI_CE,
                  labels, out_loss, out_e, reinterpret_cast<hipStream_t>(stream), out_scale);
}

extern "C" int tgemm_run_ce_grad(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                 const void* E, int64_t lde, const float* scale,
                                 const int32_t* labels, const void* B, int64_t ldb, void* C,
                                 int64_t ldc, int epilogue, void* stream) {
  if (epilogue != TGEMM_EPI_STORE_BF16 && epilogue != TGEMM_EPI_STORE_F32)
    return TGEMM_ERR_INVALID_ARG;
  if (scale == nullptr || labels == nullptr) return TGEMM_ERR_INVALID_ARG;
  const int st = tgemm_validate(transA, transB, M, N, K, E, lde, B, ldb, C, ldc, epilogue,
                                nullptr, nullptr, nullptr);
  if (st != TGEMM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // every shape on the matrix-core kernel (its loader applies the
  // rescale), without a K split
  int split = 1;
  const int cfg = choose_tile(false, (int)M, (int)N, (int)K, TGEMM_EPI_CE, &split);
  GemmParams p = {};
  p.A = static_cast<const uint16_t*>(E);
  p.B = static_cast<const uint16_t*>(B);
  p.lda = lde;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tilesM = ceil_div(M, tile_rows(cfg));
  p.tilesN = ceil_div(N, tile_cols(cfg));
  p.splitk = 1;
  p.kchunk = (int)K;
  if ((int64_t)p.tilesM * p.tilesN > kMaxWorkgroups) return TGEMM_ERR_UNSUPPORTED;
  p.groupM = p.tilesM < 4 ? p.tilesM : (p.tilesM <= 8 ? p.tilesM : 4);
  p.aligned = ((reinterpret_cast<uintptr_t>(E) | reinterpret_cast<uintptr_t>(B)) & 15) == 0 &&
              lde % 8 == 0 && ldb % 8 == 0;
  p.C = C;
  p.gscale = scale;
  p.glabels = labels;
  p.gtok = is_n(transA) ? (int)M : (int)K;
  p.gvoc = is_n(transA) ? (int)K : (int)M;
  if (verbose())
    fprintf(stderr, "tgemm: ce grad gemm %c%c M=%lld N=%lld K=%lld tile=%d\n", transA, transB,
            (long long)M, (long long)N, (long long)K, cfg);
  return status_of(launch_gemm(transA, transB, cfg,
                               epilogue == TGEMM_EPI_STORE_BF16 ? kEpiGStoreBf16 : kEpiGStoreF32,
                               p, s));
}

extern "C" int tgemm_rope_region(const void* q, int64_t ldq, int64_t P, int64_t H, int64_t D,
                                 const int64_t* pos, int64_t spos, const float* inv_freq,
                                 void* cos_out, void* sin_out, int64_t ldc, float* q_out,
                                 void* stream) {
  const int st = tgemm_validate_rope_region(q, ldq, P, H, D, pos, spos, inv_freq, cos_out,
                                            sin_out, ldc, q_out);
  if (st != TGEMM_OK) return st;
  if (verbose())
    fprintf(stderr, "tgemm: rope region P=%lld H=%lld D=%lld\n", (long long)P, (long long)H,
            (long long)D);
  const hipError_t e = launch_rope_region(static_cast<const uint16_t*>(q), ldq, P, H, D, pos, spos,
                                          inv_freq, static_cast<uint16_t*>(cos_out),
                                          static_cast<uint16_t*>(sin_out), ldc, q_out,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipErrorInvalidValue ? TGEMM_ERR_UNSUPPORTED : status_of(e);
}

// fp8 (e4m3fn) operands.  No K split, no matrix-vector or K = 1 shortcut:
// every element goes through the cast.  Two routes multiply the same
// e4m3fn values:
//  - packed (the default for large products: both tile counts at least 2,
//    every stored row 16-byte aligned with a multiple of 8 elements): a
//    pass casts each operand once into a K-contiguous code matrix, zero-
//    padded to whole tiles, in the per-stream workspace, and the fp8
//    matrix-core kernel multiplies the codes and applies the output scale;
//  - cast on load, on the bf16 kernel's register path (bf16 matrix cores,
//    each code widened back to bf16, which holds it exactly): small or
//    unaligned products, or when the workspace cannot be had.
extern "C" int tgemm_run_fp8(char transA, char transB, int64_t M, int64_t N, int64_t K,
                             const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                             int64_t ldc, int epilogue, const float* scales, void* stream) {
  const int st = tgemm_validate_fp8(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue,
                                    scales);
  if (st != TGEMM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
  // The cast costs vector work per element loaded, and a 256x256 tile loads
  // half the elements per flop of a 128x128 one: it wins from half a chip
  // of tiles up (measured on 4096x3072x4096: 237 against 248 us).
  int cfg = g_forced_tile;
  if (cfg == kTileAuto) cfg = t256 >= 128 ? kTile256 : kTile128;
  GemmParams p = {};
  p.A = static_cast<const uint16_t*>(A);
  p.B = static_cast<const uint16_t*>(B);
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tilesM = ceil_div(M, tile_rows(cfg));
  p.tilesN = ceil_div(N, tile_cols(cfg));
  p.splitk = 1;
  p.kchunk = (int)K;
  if ((int64_t)p.tilesM * p.tilesN > kMaxWorkgroups) return TGEMM_ERR_UNSUPPORTED;
  p.groupM = p.tilesM < 4 ? p.tilesM : (p.tilesM <= 8 ? p.tilesM : 4);
  p.aligned = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0 &&
              lda % 8 == 0 && ldb % 8 == 0;
  p.C = C;
  p.qscales = scales;
  const bool bf16_out = epilogue == TGEMM_EPI_STORE_BF16;
  // the stored rows' lengths (the contiguous axis)
  const int64_t colsA = is_n(transA) ? K : M, colsB = is_n(transB) ? N : K;
  // fp8 tile: the shape whose grid fills the chip best, by an estimate of
  // time = waves of 256 tiles x tile area / the shape's relative rate per
  // compute unit (measured on the fp8 kernel: 256x192 0.9 of 256x256,
  // 128x128 about 0.56).  At 4096x3072 the 256x192 tile gives exactly 256
  // tiles where 256x256 leaves 64 compute units idle.
  int f8t = kF8Tile256x256;
  if (g_forced_tile == kTile128) {
    f8t = kF8Tile128x128;
  } else if (g_forced_tile == kTileAuto) {
    double best = 0.0;
    const int cand[3] = {kF8Tile256x256, kF8Tile256x192, kF8Tile128x128};
    const double rate[3] = {1.0, 0.9, 0.56};
    for (int c = 0; c < 3; ++c) {
      const int64_t tiles =
          (int64_t)ceil_div(M, f8_tile_rows(cand[c])) * ceil_div(N, f8_tile_cols(cand[c]));
      const double t = (double)((tiles + 255) / 256) * f8_tile_rows(cand[c]) *
                       f8_tile_cols(cand[c]) / rate[c];
      if (c == 0 || t < best) {
        best = t;
        f8t = cand[c];
      }
    }
  }
  const int BTM = f8_tile_rows(f8t), BTN = f8_tile_cols(f8t);
  const int64_t Mp = (int64_t)ceil_div(M, BTM) * BTM, Np = (int64_t)ceil_div(N, BTN) * BTN;
  const int64_t Kp = (K + 127) / 128 * 128;
  const bool packed = g_fp8_cast_once && p.aligned && colsA % 8 == 0 && colsB % 8 == 0 &&
                      ceil_div(M, 256) >= 2 && ceil_div(N, 256) >= 2 && Kp / 2 < (1 << 23);
  if (verbose())
    fprintf(stderr,
            "tgemm: fp8 gemm %c%c M=%lld N=%lld K=%lld tile=%d grid=%dx%d aligned=%d "
            "packed=%d (%dx%d tiles)\n",
            transA, transB, (long long)M, (long long)N, (long long)K, cfg, p.tilesM, p.tilesN,
            p.aligned, packed ? 1 : 0, BTM, BTN);
  // the two code matrices, B's at a 256-byte boundary; without the memory
  // for them the product casts on load instead
  const size_t bytesA = (size_t)Mp * (size_t)Kp;
  const size_t offB = (bytesA + 255) / 256 * 256;
  Workspace w;
  if (!packed || get_workspace(kWsCached, s, offB + (size_t)Np * (size_t)Kp, &w) != TGEMM_OK)
    return status_of(
        launch_gemm(transA, transB, cfg, bf16_out ? kEpiQ8Bf16 : kEpiQ8F32, p, s));
  uint8_t* qa = static_cast<uint8_t*>(w.ptr);
  uint8_t* qb = static_cast<uint8_t*>(w.ptr) + offB;
  const PackOperand pa = {p.A, lda, is_n(transA), (int)M, (int)K, scales, qa, (int)Mp, (int)Kp};
  const PackOperand pb = {p.B, ldb, !is_n(transB), (int)N, (int)K, scales + 1, qb, (int)Np,
                          (int)Kp};
  hipError_t e = launch_q8_pack(pa, pb, s);
  if (e == hipSuccess) {
    p.A = reinterpret_cast<const uint16_t*>(qa);
    p.B = reinterpret_cast<const uint16_t*>(qb);
    p.lda = p.ldb = Kp / 2;
    p.K = (int)(Kp / 2);
    p.kchunk = p.K;
    p.tilesM = (int)(Mp / BTM);
    p.tilesN = (int)(Np / BTN);
    p.groupM = p.tilesM < 4 ? p.tilesM : (p.tilesM <= 8 ? p.tilesM : 4);
    e = launch_gemm_f8(f8t, bf16_out ? kEpiOsBf16 : kEpiOsF32, p, s);
  }
  const hipError_t r = release_workspace(w, s);
  return status_of(e != hipSuccess ? e : r);
}
