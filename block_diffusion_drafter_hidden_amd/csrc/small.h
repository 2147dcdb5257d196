// Launch interfaces of the small DFlash kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

enum PackMode : int { PACK_CONCAT = 0, PACK_GATE_UP = 1 };

struct PackArgs {
  const void* src[3];   // source segments, row-major [rows][K]
  int seg_tiles[3];     // 16-row tiles per segment
  int n_segs;
  int mode;             // PackMode
  int rope_segs;        // PACK_CONCAT: leading segments laid out as RoPE pairs
  int head_dim;
  int n_tiles_total;    // destination n-tiles
  int KT;               // k-tiles (K / kTile)
  long long K;          // source row length in elements
  void* dst;
};

struct EmbedNormArgs {
  const int* anchor_ids;
  int mask_id;
  const void* embed;
  int hidden;
  float* x;             // [rows][hidden] fp32 residual
  float* u;             // [rows][hidden] fp32 normed activations, or null (x only)
  const float* gain;
  float eps;
};

struct NormArgs {
  const float* x;
  float* u;
  const float* gain;
  int hidden;
  float eps;
  int drop_slot0;
};

hipError_t launch_pack(int bf16_dtype, const PackArgs& a, hipStream_t stream);
hipError_t launch_widen(int bf16_dtype, const void* src, float* dst, int n, hipStream_t stream);
hipError_t launch_embed_norm(int bf16_dtype, const EmbedNormArgs& a, int rows,
                             hipStream_t stream);
hipError_t launch_rmsnorm(int bf16_dtype, const NormArgs& a, int rows, hipStream_t stream);
hipError_t launch_verify_greedy(const int* draft, const int* target, int batch, int* accept,
                                int* bonus, int* emitted, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace dflash
