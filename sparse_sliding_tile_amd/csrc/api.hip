// C-ABI of libsta: argument validation, per-launch tables, dispatch.
//
// Every check happens before the first launch, so an error return leaves the
// outputs untouched.  Window tables are copied into the kernel arguments of the
// launch that uses them; nothing is kept between calls.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "kernels.h"

using namespace sta;

namespace {

int to_status(hipError_t e) { return e == hipSuccess ? STA_OK : STA_ERR_HIP; }

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

int make_geometry(sta_dim3 latent, sta_dim3 tile, Geometry* g) {
  if (latent.t < 1 || latent.h < 1 || latent.w < 1 || tile.t < 1 || tile.h < 1 || tile.w < 1)
    return STA_ERR_ARG;
  // A latent that is not a whole number of tiles is padded up (ceil grid).
  const int64_t n0 = (latent.t + (int64_t)tile.t - 1) / tile.t;
  const int64_t n1 = (latent.h + (int64_t)tile.h - 1) / tile.h;
  const int64_t n2 = (latent.w + (int64_t)tile.w - 1) / tile.w;
  const int64_t L = (int64_t)tile.t * tile.h * tile.w;
  const int64_t S = n0 * n1 * n2 * L;
  if (L >= (1ll << 31) || S >= (1ll << 31)) return STA_ERR_TOO_LARGE;
  // Clamped window widths travel to the kernels as 16-bit values.
  if (n0 > kMaxGridTiles || n1 > kMaxGridTiles || n2 > kMaxGridTiles) return STA_ERR_TOO_LARGE;
  g->T = latent.t;
  g->H = latent.h;
  g->W = latent.w;
  g->t = tile.t;
  g->h = tile.h;
  g->w = tile.w;
  g->n0 = (int)n0;
  g->n1 = (int)n1;
  g->n2 = (int)n2;
  g->L = (int)L;
  g->S = (int)S;
  g->Sr = latent.t * latent.h * latent.w;
  g->ntiles = g->n0 * g->n1 * g->n2;
  g->padded = (latent.t % tile.t || latent.h % tile.h || latent.w % tile.w) ? 1 : 0;
  g->fw = make_fastdiv((uint32_t)tile.w);
  g->fhw = make_fastdiv((uint32_t)(tile.h * tile.w));
  return STA_OK;
}

// Clamps windows to the grid (w' = min(w, n)) and orders heads for launch:
// heaviest window first (stable), then dealt round-robin over the 8 XCD slots
// so that each XCD's contiguous run of work items gets a similar load.
int make_heads(const int32_t* win, int64_t Hh, const Geometry& g, HeadTable* ht) {
  if (win == nullptr || Hh < 1) return STA_ERR_ARG;
  if (Hh > STA_MAX_HEADS) return STA_ERR_UNSUPPORTED;
  memset(ht, 0, sizeof(*ht));
  const int n[3] = {g.n0, g.n1, g.n2};
  std::vector<int64_t> weight(Hh);
  for (int64_t h = 0; h < Hh; ++h) {
    weight[h] = 1;
    for (int d = 0; d < 3; ++d) {
      const int32_t w = win[3 * h + d];
      if (w < 1) return STA_ERR_WINDOW;
      ht->wp[h][d] = (uint16_t)window_width(w, n[d]);
      weight[h] *= ht->wp[h][d];
    }
  }
  std::vector<int> idx(Hh);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return weight[a] > weight[b]; });
  int pos = 0;
  for (int x = 0; x < 8; ++x)
    for (int64_t j = x; j < Hh; j += 8) ht->order[pos++] = (uint8_t)idx[j];
  return STA_OK;
}

int elem_bytes(sta_dtype dt) { return dt == STA_BF16 ? 2 : (dt == STA_F32 ? 4 : 0); }

int check_sizes(int64_t B, int64_t Hh, int64_t D, const Geometry& g) {
  if (B < 1 || Hh < 1 || D < 1) return STA_ERR_ARG;
  if (B * Hh * (int64_t)g.ntiles >= (1ll << 31) / 4) return STA_ERR_TOO_LARGE;
  return STA_OK;
}

}  // namespace

extern "C" {

const char* sta_strerror(int code) {
  switch (code) {
    case STA_OK: return "success";
    case STA_ERR_ARG: return "invalid argument (null pointer, non-positive size or scale)";
    case STA_ERR_NOT_TILE_MULTIPLE: return "latent is not an integer multiple of the tile";
    case STA_ERR_WINDOW: return "window entries must be at least one tile";
    case STA_ERR_UNSUPPORTED: return "head_dim, tile volume, head count or dtype not supported";
    case STA_ERR_ALIGN: return "tensor pointer is not 16-byte aligned";
    case STA_ERR_HIP: return "HIP runtime error at launch";
    case STA_ERR_WORKSPACE: return "workspace missing or too small";
    case STA_ERR_TOO_LARGE: return "size exceeds the 32-bit index range of the kernels";
    default: return "unknown error code";
  }
}

static int tile_copy(const void* src, void* dst, int64_t B, int64_t Hh, int64_t D,
                     sta_dim3 latent, sta_dim3 tile, sta_dtype dt, void* stream, bool to_tm) {
  Geometry g;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if (!src || !dst) return STA_ERR_ARG;
  if ((st = check_sizes(B, Hh, D, g))) return st;
  const int eb = elem_bytes(dt);
  if (!eb) return STA_ERR_UNSUPPORTED;
  if (misaligned(src) || misaligned(dst)) return STA_ERR_ALIGN;
  if (D * eb >= (1ll << 24)) return STA_ERR_TOO_LARGE;
  return to_status(launch_tile_copy(src, dst, B * Hh, D * eb, g, to_tm, (hipStream_t)stream));
}

int sta_tile_reorder(const void* x, void* y, int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                     sta_dim3 tile, sta_dtype dt, void* stream) {
  return tile_copy(x, y, B, Hh, D, latent, tile, dt, stream, true);
}

int sta_tile_unreorder(const void* y, void* x, int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                       sta_dim3 tile, sta_dtype dt, void* stream) {
  return tile_copy(y, x, B, Hh, D, latent, tile, dt, stream, false);
}

int64_t sta_tile_pairs_count(sta_dim3 latent, sta_dim3 tile, const int32_t* win_host, int64_t Hh,
                             int transpose) {
  if (transpose != 0 && transpose != 1) return STA_ERR_ARG;
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  int64_t n = 0;
  for (int64_t h = 0; h < Hh; ++h) n += (int64_t)g.ntiles * ht.wp[h][0] * ht.wp[h][1] * ht.wp[h][2];
  return n;
}

static void fill_offsets(int64_t* off, const Geometry& g, const HeadTable& ht, int64_t Hh) {
  off[0] = 0;
  for (int64_t h = 0; h < Hh; ++h)
    off[h + 1] = off[h] + (int64_t)g.ntiles * ht.wp[h][0] * ht.wp[h][1] * ht.wp[h][2];
}

int sta_tile_pairs(int32_t* pairs_dev, int64_t* head_offsets_host, sta_dim3 latent, sta_dim3 tile,
                   const int32_t* win_host, int64_t Hh, int transpose, void* stream) {
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  if (!pairs_dev) return STA_ERR_ARG;
  if (Hh * (int64_t)g.ntiles >= (1ll << 31)) return STA_ERR_TOO_LARGE;
  if (head_offsets_host) fill_offsets(head_offsets_host, g, ht, Hh);
  return to_status(launch_tile_pairs(pairs_dev, g, ht, (int)Hh, transpose ? 1 : 0,
                                     (hipStream_t)stream));
}

int sta_tile_pairs_host(int32_t* pairs_host, int64_t* head_offsets_host, sta_dim3 latent,
                        sta_dim3 tile, const int32_t* win_host, int64_t Hh, int transpose) {
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  if (!pairs_host) return STA_ERR_ARG;
  if (head_offsets_host) fill_offsets(head_offsets_host, g, ht, Hh);
  host_tile_pairs(pairs_host, g, ht, (int)Hh, transpose ? 1 : 0);
  return STA_OK;
}

static int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hh, int64_t D, const Geometry& g, const HeadTable& ht,
                        float scale, sta_dtype dt, void* stream) {
  if (!q || !k || !v || !o) return STA_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return STA_ERR_ARG;
  int st = check_sizes(B, Hh, D, g);
  if (st) return st;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return STA_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  if (dt == STA_BF16) {
    if (!fwd_bf16_supported((int)D, g)) return STA_ERR_UNSUPPORTED;
    return to_status(launch_fwd_bf16((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                     (uint16_t*)o, lse, g, ht, (int)B, (int)Hh, (int)D, scale, s));
  }
  if (dt == STA_F32) {
    if (D != 32 && D != 64 && D != 128) return STA_ERR_UNSUPPORTED;
    return to_status(launch_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o,
                                    lse, g, ht, (int)B, (int)Hh, (int)D, scale, s));
  }
  return STA_ERR_UNSUPPORTED;
}

int sta_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile, const int32_t* win_host,
                float scale, sta_dtype dt, void* stream) {
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  return forward_impl(q, k, v, o, lse, B, Hh, D, g, ht, scale, dt, stream);
}

int sta_forward_raster(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                       const int32_t* win_host, float scale, sta_dtype dt, void* stream) {
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  if (!q || !k || !v || !o) return STA_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return STA_ERR_ARG;
  if ((st = check_sizes(B, Hh, D, g))) return st;
  if (dt != STA_BF16 || !fwd_raster_supported((int)D, g)) return STA_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return STA_ERR_ALIGN;
  return to_status(launch_fwd_bf16_raster((const uint16_t*)q, (const uint16_t*)k,
                                          (const uint16_t*)v, (uint16_t*)o, lse, g, ht, (int)B,
                                          (int)Hh, (int)D, scale, (hipStream_t)stream));
}

size_t sta_backward_workspace_bytes(int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                                    sta_dim3 tile, sta_dtype dt) {
  (void)D;
  Geometry g;
  if (B < 1 || Hh < 1 || make_geometry(latent, tile, &g) != STA_OK) return 0;
  const size_t S = (size_t)g.S;
  // Per tile-major row: Dl = <dO, O> and LSE * log2(e), fp32.  The bf16 path
  // adds a key-tile order per head (int32).
  size_t bytes = 2 * (size_t)B * Hh * S * sizeof(float);
  if (dt == STA_BF16) bytes += (size_t)Hh * g.ntiles * sizeof(int32_t);
  return bytes;
}

int sta_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                 int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                 const int32_t* win_host, float scale, sta_dtype dt, void* stream) {
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return STA_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return STA_ERR_ARG;
  if ((st = check_sizes(B, Hh, D, g))) return st;
  if (!workspace || ws_bytes < sta_backward_workspace_bytes(B, Hh, D, latent, tile, dt))
    return STA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return STA_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  if (dt == STA_BF16) {
    if (!bwd_bf16_supported((int)D, g)) return STA_ERR_UNSUPPORTED;
    return to_status(launch_bwd_bf16(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
        (const uint16_t*)dout, lse, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, (float*)workspace,
        g, ht, (int)B, (int)Hh, (int)D, scale, s));
  }
  if (dt == STA_F32) {
    if (D != 32 && D != 64 && D != 128) return STA_ERR_UNSUPPORTED;
    return to_status(launch_bwd_f32((const float*)q, (const float*)k, (const float*)v,
                                    (const float*)o, (const float*)dout, lse, (float*)dq,
                                    (float*)dk, (float*)dv, (float*)workspace, g, ht, (int)B,
                                    (int)Hh, (int)D, scale, s));
  }
  return STA_ERR_UNSUPPORTED;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Static scratch for sta_backward_noalloc.  Each GPU the library runs on holds
// its own copy of this array until the process ends.  In host code the name
// is only a stand-in: the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current, looked up once per device and
// kept in noalloc_scratch[].
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[STA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag noalloc_once[kMaxDevices];
void* noalloc_scratch[kMaxDevices];
hipError_t noalloc_status[kMaxDevices];

// The current device's copy of `scratch`, or nullptr (with *err set).
void* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(noalloc_once[dev], [dev]() {
    void* ptr = nullptr;
    noalloc_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    noalloc_scratch[dev] = noalloc_status[dev] == hipSuccess ? ptr : nullptr;
  });
  *err = noalloc_status[dev];
  return noalloc_scratch[dev];
}
}  // namespace

extern "C" {

int sta_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                         const int32_t* win_host, float scale, sta_dtype dt, void* stream) {
  // Every argument check of sta_backward runs first (with the workspace
  // replaced by the static array), so a rejected call touches no device.
  Geometry g;
  HeadTable ht;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if ((st = make_heads(win_host, Hh, g, &ht))) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return STA_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return STA_ERR_ARG;
  if ((st = check_sizes(B, Hh, D, g))) return st;
  const size_t need = sta_backward_workspace_bytes(B, Hh, D, latent, tile, dt);
  if (need == 0 || need > (size_t)STA_NOALLOC_SCRATCH_BYTES) return STA_ERR_TOO_LARGE;
  hipError_t e = hipSuccess;
  void* ws = scratch_for_current_device(&e);
  if (ws == nullptr) return STA_ERR_HIP;
  return sta_backward(q, k, v, o, dout, lse, dq, dk, dv, ws, need, B, Hh, D, latent, tile, win_host,
                      scale, dt, stream);
}

int sta_dense_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t Hh, int64_t S, int64_t D, float scale, sta_dtype dt, void* stream) {
  if (S < 1 || S >= (1ll << 31)) return S < 1 ? STA_ERR_ARG : STA_ERR_TOO_LARGE;
  // Dense attention is the window rule on a 1 x 1 x (S/Lt) grid of Lt-token
  // tiles with a window spanning the whole grid.
  int64_t Lt;
  if (dt == STA_BF16) {
    if (S % 384 == 0) Lt = 384;
    else if (S % 128 == 0) Lt = 128;
    else if (S % 32 == 0) Lt = 32;
    else return STA_ERR_UNSUPPORTED;
  } else {
    Lt = S;
  }
  Geometry g;
  HeadTable ht;
  int st = make_geometry(sta_dim3{1, 1, (int32_t)S}, sta_dim3{1, 1, (int32_t)Lt}, &g);
  if (st) return st;
  if (Hh < 1) return STA_ERR_ARG;
  if (Hh > STA_MAX_HEADS) return STA_ERR_UNSUPPORTED;
  std::vector<int32_t> win(3 * Hh);
  for (int64_t h = 0; h < Hh; ++h) {
    win[3 * h] = 1;
    win[3 * h + 1] = 1;
    win[3 * h + 2] = g.n2;
  }
  if ((st = make_heads(win.data(), Hh, g, &ht))) return st;
  return forward_impl(q, k, v, o, lse, B, Hh, D, g, ht, scale, dt, stream);
}

static_assert(STA_MAX_CANDIDATES == kMaxCandidates, "candidate limit");

size_t sta_window_mass_workspace_bytes(int64_t B, int64_t Hh, sta_dim3 latent, sta_dim3 tile,
                                       int64_t n_cand) {
  Geometry g;
  if (B < 1 || Hh < 1 || n_cand < 1 || make_geometry(latent, tile, &g) != STA_OK) return 0;
  // Two fp32 log-sum-exp vectors over the tile-major rows (full window, last
  // candidate), then one fp32 partial sum per (candidate, sequence, 32 rows).
  const size_t rows = (size_t)B * Hh * (size_t)g.S;
  return 2 * rows * sizeof(float) + (size_t)n_cand * B * Hh * ((g.S + 31) / 32) * sizeof(float);
}

int sta_window_mass(const void* q, const void* k, float* mass, void* workspace, size_t ws_bytes,
                    int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                    const int32_t* cand_host, int64_t n_cand, float scale, sta_dtype dt,
                    void* stream) {
  Geometry g;
  int st = make_geometry(latent, tile, &g);
  if (st) return st;
  if (!q || !k || !mass || !cand_host || n_cand < 1) return STA_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return STA_ERR_ARG;
  if ((st = check_sizes(B, Hh, D, g))) return st;
  if (Hh > STA_MAX_HEADS || n_cand > STA_MAX_CANDIDATES) return STA_ERR_UNSUPPORTED;
  if (dt == STA_BF16) {
    if (!fwd_bf16_supported((int)D, g)) return STA_ERR_UNSUPPORTED;
  } else if (dt == STA_F32) {
    if (D != 32 && D != 64 && D != 128) return STA_ERR_UNSUPPORTED;
  } else {
    return STA_ERR_UNSUPPORTED;
  }
  if (!workspace || ws_bytes < sta_window_mass_workspace_bytes(B, Hh, latent, tile, n_cand))
    return STA_ERR_WORKSPACE;
  if (misaligned(q) || misaligned(k) || misaligned(workspace)) return STA_ERR_ALIGN;
  // Every table is built (and every window checked) before the first launch.
  std::vector<int32_t> win(3 * (size_t)Hh);
  for (int64_t h = 0; h < Hh; ++h) {
    win[3 * h] = g.n0;
    win[3 * h + 1] = g.n1;
    win[3 * h + 2] = g.n2;
  }
  HeadTable full;
  if ((st = make_heads(win.data(), Hh, g, &full))) return st;
  std::vector<HeadTable> cands((size_t)n_cand);
  for (int64_t c = 0; c < n_cand; ++c) {
    for (int64_t h = 0; h < Hh; ++h)
      for (int d = 0; d < 3; ++d) win[3 * h + d] = cand_host[3 * c + d];
    if ((st = make_heads(win.data(), Hh, g, &cands[c]))) return st;
  }
  const hipStream_t s = (hipStream_t)stream;
  float* lse_full = (float*)workspace;
  float* lse_win = lse_full + (size_t)B * Hh * g.S;
  if (dt == STA_BF16) {
    // one pass: the full window, every candidate's share under it
    MassArgs ma{};
    ma.partial = lse_win + (size_t)B * Hh * g.S;
    ma.lse_last = lse_win;
    ma.ncand = (int)n_cand;
    for (int64_t c = 0; c < n_cand; ++c)
      for (int d = 0; d < 3; ++d) ma.w[c][d] = cands[c].wp[0][d];  // clamped, same for all heads
    hipError_t e = launch_mass_bf16((const uint16_t*)q, (const uint16_t*)k, lse_full, ma, g, full,
                                    (int)B, (int)Hh, (int)D, scale, s);
    if (e == hipSuccess) e = launch_mass_reduce(ma.partial, mass, g, (int)n_cand, B * Hh, s);
    return to_status(e);
  }
  // fp32 debug path: a normaliser pass per window, then the mean of
  // exp(LSE_win - LSE_full)
  hipError_t e = launch_fwd_f32((const float*)q, (const float*)k, (const float*)k, nullptr,
                                lse_full, g, full, (int)B, (int)Hh, (int)D, scale, s);
  for (int64_t c = 0; c < n_cand && e == hipSuccess; ++c) {
    e = launch_fwd_f32((const float*)q, (const float*)k, (const float*)k, nullptr, lse_win, g,
                       cands[c], (int)B, (int)Hh, (int)D, scale, s);
    if (e == hipSuccess) e = launch_mass(lse_win, lse_full, mass + c * B * Hh, g, B * Hh, s);
  }
  return to_status(e);
}

}  // extern "C"
