/*
 * libsta: Sliding Tile Attention (STA) on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages, cited by title and section):
 *   [STA-abs]   "Sliding Tile Attention" (arXiv 2502.04507), abstract as printed
 *               on the gptget.net summary page: softmax attention where every
 *               query attends only to keys inside a local 3D (T,H,W) window, the
 *               window being taken tile by tile instead of token by token.
 *   [STA-meth]  same page, sections on the core innovation and method details:
 *               the latent is cut into non-overlapping space-time tiles made
 *               contiguous in the sequence; every (query tile, key tile) block is
 *               either fully computed or skipped, never half masked; every head
 *               has its own window size.
 *   [STA-rebut] "Fast Video Generation with Sliding Tile Attention", OpenReview
 *               rebuttal, answer on input resolution: tile (6,8,8); the latent
 *               should be an integer multiple of the tile, and other latents are
 *               handled by padding with masking.
 *
 * Conventions shared by every entry point
 *   - Shapes are (T, H, W) triples, W fastest.  A raster token r = (tau*H+y)*W+x.
 *   - Tensors are contiguous [B, Hh, S, D] (D innermost), element type bf16
 *     (STA_BF16) or fp32 (STA_F32, the fp32 debug instance).  Raster-order
 *     tensors have S = T*H*W rows; tile-major tensors have S' = n0*n1*n2*L rows.
 *     LSE is fp32 [B, Hh, S'] in tile-major order.
 *   - Tile-major order: tiles in raster order over the tile grid
 *     n = (ceil(T/t), ceil(H/h), ceil(W/w)), tokens in raster order inside a
 *     tile; tile number a occupies sequence positions [a*L, (a+1)*L), L = t*h*w.
 *   - Padding with masking [STA-rebut]: when the latent is not a whole number of
 *     tiles, the tile grid covers the latent padded up to whole tiles (S' > S).
 *     Tile-major positions whose (t, h, w) coordinate lies outside the latent
 *     are padding: they are never keys, and O, LSE, dQ, dK and dV are written as
 *     zero there.  Their contents in q, k, v and dout may be any finite values
 *     (sta_tile_reorder writes zeros): the kernels mask padding keys and
 *     queries with selects, so even contents whose products overflow fp32
 *     affect no other row.
 *   - Window of a head: (wt, wh, ww) in tiles, each >= 1.  Along a dimension with
 *     n tiles, w' = min(w, n) and the window of query tile q covers tiles
 *     [s, s + w') with s = clamp(q - floor(w'/2), 0, n - w'): the centre is
 *     clamped so the window always stays inside the tile grid and always holds
 *     w' tiles.  The window table is a HOST array int32 [Hh][3], read during the
 *     call only (the caller may free it on return); at most STA_MAX_HEADS heads.
 *   - All tensor pointers are device memory owned by the caller, 16-byte aligned.
 *     The library never allocates device memory.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Kernel
 *     launches are asynchronous: a return of STA_OK means the work was queued.
 *   - Return value: STA_OK (0) or a negative STA_ERR_* code.  Every argument is
 *     validated before anything is launched; on an error nothing is launched and
 *     no output is touched.  The only mutable global state is the static
 *     scratch of sta_backward_noalloc (see there); every other call is
 *     thread-safe; calls that write the same buffers must be ordered by the caller.
 */
#ifndef STA_H_
#define STA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility: exactly the functions below
 * are exported. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

typedef struct {
  int32_t t, h, w;
} sta_dim3;

typedef enum { STA_BF16 = 0, STA_F32 = 1 } sta_dtype;

enum {
  STA_OK = 0,
  STA_ERR_ARG = -1,               /* null pointer, non-positive size, bad scale */
  STA_ERR_NOT_TILE_MULTIPLE = -2, /* reserved: every call pads such latents with masking */
  STA_ERR_WINDOW = -3,            /* a window entry < 1 */
  STA_ERR_UNSUPPORTED = -4,       /* head_dim, tile volume or dtype not built */
  STA_ERR_ALIGN = -5,             /* a tensor pointer not 16-byte aligned */
  STA_ERR_HIP = -6,               /* the HIP runtime reported an error at launch */
  STA_ERR_WORKSPACE = -7,         /* workspace missing or smaller than required */
  STA_ERR_TOO_LARGE = -8          /* a size exceeds the kernels' index range (32-bit rows,
                                     at most 65535 tiles along each grid dimension) */
};

#define STA_MAX_HEADS 256
#define STA_MAX_CANDIDATES 8 /* candidate windows per sta_window_mass call */
#define STA_NOALLOC_SCRATCH_BYTES (32u << 20) /* static scratch of sta_backward_noalloc */

/* Human-readable text for a return code (static storage). */
const char* sta_strerror(int code);

/* Tile reorder [STA-meth], raster -> tile-major along S:
 *   y[b, hh, pi(r), :] = x[b, hh, r, :]
 * where pi(r) is the tile-major position of raster token r.  x is
 * [B, Hh, S, D], y is [B, Hh, S', D] (S' = S for a whole-tile latent), distinct
 * buffers of type dt.  A bit-exact copy; padding rows of y are set to zero. */
int sta_tile_reorder(const void* x, void* y, int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                     sta_dim3 tile, sta_dtype dt, void* stream);

/* Inverse of sta_tile_reorder: x[b, hh, r, :] = y[b, hh, pi(r), :] for the S
 * raster tokens (padding rows of y are not read). */
int sta_tile_unreorder(const void* y, void* x, int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                       sta_dim3 tile, sta_dtype dt, void* stream);

/* Number of (query tile, key tile) pairs over all heads: sum_h N_t * prod_d w'_d
 * ([STA-meth]: the blocks that are computed), for the list sta_tile_pairs writes
 * with the same transpose flag (0: query-major, 1: key-major; both orders hold
 * the same pairs, so the count is the same).  Host only; returns a negative
 * STA_ERR_* code on bad arguments (STA_ERR_ARG for a flag other than 0 or 1). */
int64_t sta_tile_pairs_count(sta_dim3 latent, sta_dim3 tile, const int32_t* win_host, int64_t Hh,
                             int transpose);

/* Canonical tile-pair list, written by a kernel that uses the same window
 * function as sta_forward / sta_backward.  Tiles are numbered in raster order
 * over the tile grid.  pairs_dev: device int32 [count][2] of (q_tile, k_tile).
 * transpose = 0: ordered by head, then query tile, then key tile (the forward's
 * view); transpose = 1: by head, then key tile, then query tile (the set of query
 * tiles whose window holds a key tile: the backward's view).  head_offsets_host
 * (nullable): host int64 [Hh + 1], prefix offsets of each head's pairs, filled
 * before return. */
int sta_tile_pairs(int32_t* pairs_dev, int64_t* head_offsets_host, sta_dim3 latent, sta_dim3 tile,
                   const int32_t* win_host, int64_t Hh, int transpose, void* stream);

/* Same list computed on the host into host memory (pairs_host int32 [count][2]),
 * with the same window function compiled for the CPU. */
int sta_tile_pairs_host(int32_t* pairs_host, int64_t* head_offsets_host, sta_dim3 latent,
                        sta_dim3 tile, const int32_t* win_host, int64_t Hh, int transpose);

/* STA forward [STA-abs]: for every (b, hh) and query position i of query tile a,
 *   O_i = sum_j softmax_j(scale * <q_i, k_j>) v_j   over key positions j whose
 *   tile lies in the window of a,   LSE_i = ln sum_j exp(scale * <q_i, k_j>).
 * q, k, v, o: [B, Hh, S', D] in TILE-MAJOR order (see sta_tile_reorder).
 * lse: fp32 [B, Hh, S'] or NULL.  scale > 0 (usually 1/sqrt(D)).
 * STA_BF16: bf16 in/out, fp32 accumulation, MFMA; needs D in {64, 128},
 * L % 32 == 0 and, for a latent that is not a whole number of tiles,
 * L <= 2^20.  STA_F32: fp32 in/out, fp32 arithmetic; needs D in {32, 64, 128}. */
int sta_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile, const int32_t* win_host,
                float scale, sta_dtype dt, void* stream);

/* STA forward on raster-order tensors ([STA-abs] attention over the tile
 * window, with [STA-meth]'s tile-contiguous order used only inside the
 * kernel): the tile reorder of q, k, v and the unreorder of o (and lse)
 * folded into the kernel's own loads and stores, so
 * one launch replaces reorder x3 + sta_forward + unreorder with the same
 * arithmetic in the same order (outputs bit-identical to that sequence).
 * q, k, v, o: bf16 [B, Hh, T*H*W, D] in raster order (W fastest); lse: fp32
 * [B, Hh, T*H*W] raster or NULL.  A latent that is not a whole number of
 * tiles is padded with masking as in sta_forward: the raster tensors hold
 * only the T*H*W real tokens (padding positions have no rows, are never
 * keys and produce no output).  Needs STA_BF16 with D in {64, 128},
 * L % 32 == 0, the tile width a multiple of 512 / D and
 * L <= 1024 * 512 / D, i.e. 4096 tokens for D = 128 and 8192 for D = 64
 * (STA_ERR_UNSUPPORTED otherwise).  Other arguments as sta_forward. */
int sta_forward_raster(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                       const int32_t* win_host, float scale, sta_dtype dt, void* stream);

/* Bytes of device workspace sta_backward needs: 8*B*Hh*S' for per-row
 * statistics (fp32: Dl, held negated by the bf16 path, and LSE*log2(e); on
 * padding rows 0 and +inf) plus,
 * for STA_BF16, 4*Hh*n0*n1*n2 for a per-head order of the key tiles.  0 for
 * invalid sizes. */
size_t sta_backward_workspace_bytes(int64_t B, int64_t Hh, int64_t D, sta_dim3 latent,
                                    sta_dim3 tile, sta_dtype dt);

/* STA backward: the exact gradient of sta_forward (the pages name fine-tuning
 * with STA [STA-meth], which needs it).  With P the window-masked softmax,
 *   Dl_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - Dl_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   dV_j = sum_i P_ij dO_i.
 * Inputs q, k, v, o, dout (tile-major, type dt) and lse (fp32, from
 * sta_forward); outputs dq, dk, dv (tile-major, type dt), fully overwritten.
 * Sizes as sta_forward: STA_BF16 needs D in {64, 128}, L % 32 == 0 and, for a
 * latent that is not a whole number of tiles, L <= 2^20 (STA_ERR_UNSUPPORTED
 * otherwise).
 * workspace: device memory of at least sta_backward_workspace_bytes(), owned by
 * the caller, contents on entry irrelevant. */
int sta_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                 int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                 const int32_t* win_host, float scale, sta_dtype dt, void* stream);

/* sta_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the workspace replaced by a static
 * device array of STA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds
 * on each GPU it runs on until the process ends.  It calls no hipMalloc,
 * hipFree or other allocating routine.  Arguments as sta_backward, without
 * workspace and ws_bytes; sizes whose workspace
 * (sta_backward_workspace_bytes) exceeds the array are refused with
 * STA_ERR_TOO_LARGE before anything is launched (2*B*Hh*S' fp32 row
 * statistics plus the bf16 path's key-tile order must fit: about 4.19 M
 * tile-major rows over all (b, head)).  The first call on a device looks the
 * array's address up (hipGetSymbolAddress); STA_ERR_HIP if that fails.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, or several host threads) race and must be
 * serialised by the caller.  Nothing in the array needs to start at zero:
 * every value the kernels read from it is written earlier in the same call. */
int sta_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                         const int32_t* win_host, float scale, sta_dtype dt, void* stream);

/* Dense softmax attention over all S keys: the full-attention baseline STA is
 * compared with ([STA-abs] compares with FlashAttention).  Same kernel family
 * and layout as sta_forward; S % 32 == 0 for STA_BF16. */
int sta_dense_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t Hh, int64_t S, int64_t D, float scale, sta_dtype dt, void* stream);

/* Bytes of device workspace sta_window_mass needs: 8*B*Hh*S' (two fp32
 * log-sum-exp vectors over the tile-major rows) plus 4*n_cand*B*Hh*ceil(S'/32)
 * (per-block partial sums).  0 for invalid sizes. */
size_t sta_window_mass_workspace_bytes(int64_t B, int64_t Hh, sta_dim3 latent, sta_dim3 tile,
                                       int64_t n_cand);

/* Attention mass of candidate windows, the measurement side of the per-head
 * window search ([STA-meth]: each head gets its own window, configured
 * automatically; [STA-abs]: attention concentrates in local 3D windows).
 * For query row i of (batch b, head h), with s_ij = scale <q_i, k_j> over ALL
 * real keys j, the share of the full softmax that candidate window w keeps is
 *   mass_i(w) = sum_{j in w} exp(s_ij) / sum_j exp(s_ij)
 *             = exp(LSE_w,i - LSE_full,i),
 * and mass[c][b][h] (fp32, device, n_cand*B*Hh values, fully overwritten) is
 * its mean over the real query rows of (b, h) for window cand_host[c].
 * q, k: tile-major [B, Hh, S', D] of type dt (as for sta_forward; V is not
 * needed).  cand_host: host int32 [n_cand][3] windows in tiles, each >= 1,
 * clamped to the grid, the same for every head; read during the call;
 * 1 <= n_cand <= STA_MAX_CANDIDATES (STA_ERR_UNSUPPORTED above).
 * workspace: device memory of at least sta_window_mass_workspace_bytes(),
 * caller-owned, contents on entry irrelevant; on return it starts with the
 * per-row statistics: fp32 [B, Hh, S'] LSE of the full window, then fp32
 * [B, Hh, S'] LSE of the last candidate (natural log, tile-major rows, 0 on
 * padding rows).  STA_BF16 does the work in one pass over the full window
 * (Q K^T and the normaliser only; every candidate's share is summed under the
 * shared running maximum), STA_F32 in one normaliser pass per window.
 * Errors as sta_forward, plus STA_ERR_WORKSPACE. */
int sta_window_mass(const void* q, const void* k, float* mass, void* workspace, size_t ws_bytes,
                    int64_t B, int64_t Hh, int64_t D, sta_dim3 latent, sta_dim3 tile,
                    const int32_t* cand_host, int64_t n_cand, float scale, sta_dtype dt,
                    void* stream);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* STA_H_ */
