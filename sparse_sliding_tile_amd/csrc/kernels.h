// Internal launcher declarations shared by the kernel sources and the C-ABI.
#pragma once

#include "sta_common.h"

namespace sta {

// Reorder (to_tile_major) or unreorder of BH = B*Hh sequences of S rows.
hipError_t launch_tile_copy(const void* src, void* dst, int64_t BH, int64_t row_bytes,
                            const Geometry& g, bool to_tile_major, hipStream_t stream);

hipError_t launch_tile_pairs(int32_t* out, const Geometry& g, const HeadTable& ht, int Hh,
                             int transpose, hipStream_t stream);
void host_tile_pairs(int32_t* out, const Geometry& g, const HeadTable& ht, int Hh, int transpose);

// fp32 debug instance (D in {32, 64, 128}).  o == nullptr computes the LSE
// alone (v is then not read).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                          float scale, hipStream_t stream);
hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* dl, const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                          float scale, hipStream_t stream);

// bf16 MFMA instance (D in {64, 128}, L % 32 == 0, and L <= 2^20 for a
// padded latent).
bool fwd_bf16_supported(int D, const Geometry& g);
hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                           int D, float scale, hipStream_t stream);
// The same forward on raster-order q, k, v, o and lse (the reorder folded into
// the kernel's loads and stores): latents whose tile width is a multiple of
// 512 / D rows.
bool fwd_raster_supported(int D, const Geometry& g);
hipError_t launch_fwd_bf16_raster(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* o, float* lse, const Geometry& g, const HeadTable& ht,
                                  int B, int Hh, int D, float scale, hipStream_t stream);
// Window mass of up to kMaxCandidates candidate windows in one pass over the
// full window (Q K^T and the softmax normaliser only, V not read): per query
// row, the full normaliser l and, per candidate c, the part l_c of it whose
// key tiles lie in window c, under one running maximum; l_c / l is the row's
// mass.  Per-wave sums of the row masses go to partial[c][b*Hh+h][S/32],
// LSE_full to lse, the last candidate's LSE to lse_last (both per row).
constexpr int kMaxCandidates = 8;
struct MassArgs {
  float* partial;
  float* lse_last;
  int ncand;
  uint16_t w[kMaxCandidates][3];  // clamped to the grid
};
hipError_t launch_mass_bf16(const uint16_t* q, const uint16_t* k, float* lse, const MassArgs& ma,
                            const Geometry& g, const HeadTable& ht_full, int B, int Hh, int D,
                            float scale, hipStream_t stream);
// mass[c][bh] = (sum of partial[c][bh][0 .. S/32)) / real rows.
hipError_t launch_mass_reduce(const float* partial, float* mass, const Geometry& g, int ncand,
                              int64_t BH, hipStream_t stream);
bool bwd_bf16_supported(int D, const Geometry& g);
hipError_t launch_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const uint16_t* dout, const float* lse,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dl,
                           const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                           float scale, hipStream_t stream);

// mass[bh] = mean over the real rows of sequence bh of exp(lse_win - lse_full).
hipError_t launch_mass(const float* lse_win, const float* lse_full, float* mass, const Geometry& g,
                       int64_t BH, hipStream_t stream);

}  // namespace sta
