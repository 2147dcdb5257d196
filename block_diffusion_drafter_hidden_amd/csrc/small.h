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

struct EmbedArgs {
  const int* anchor_ids;  // [batch]
  int mask_id;
  const void* embed;      // [vocab][hidden] model dtype
  int hidden;
  int rpr;                // rows per request (16, or 32 for a 32-token block)
  float* x;               // residual stream, fp32 fragment layout (rows = batch * rpr)
  const float* gamma;     // first layer's attention RMSNorm gain [hidden]
  void* xg;               // x * gamma: pair fragment layout (bf16 models), else as x
  float* ssq;             // [rows] sum of squares of each row
};

hipError_t launch_pack(int bf16_dtype, const PackArgs& a, hipStream_t stream);
hipError_t launch_widen(int bf16_dtype, const void* src, float* dst, int n, hipStream_t stream);
// norms[r] = Euclidean norm of row r of the row-major [rows][cols] matrix w (model dtype),
// *out_max = the largest of them.
hipError_t launch_row_norm_max(int bf16_dtype, const void* w, int rows, int cols, float* norms,
                               float* out_max, hipStream_t stream);
hipError_t launch_embed(int bf16_dtype, const EmbedArgs& a, int rows, hipStream_t stream);
// Row-major fp32 [rows][cols] -> dst = src * gamma, in the pair fragment layout (hilo = 1,
// bf16 models) or the fp32 fragment layout with kPer 4 (fp32 models), and ssq[r] = sum of
// squares of row r (the inputs of an RMSNorm-folded GEMM); cols % 32 == 0.
hipError_t launch_rows_to_fragments(const float* src, int rows, int cols, int hilo,
                                    const float* gamma, void* dst, float* ssq,
                                    hipStream_t stream);
// Input-fusion prefill helpers: the rows' norm inputs (padding rows >= n_valid zeroed) and
// the cached context of each 16-row group, ctx_lens[seq] + r0 + 16 g.
hipError_t launch_prefill_rows(int bf16_dtype, float* x, int rows, int n_valid, int hidden,
                               const float* gamma, void* xg, float* ssq, hipStream_t stream);
hipError_t launch_prefill_groups(const int* ctx_lens, int seq, int r0, int groups,
                                 int* group_ctx, hipStream_t stream);
// Block of nb tokens: draft [batch][nb - 1], target [batch][nb], emitted [batch][nb].
hipError_t launch_verify_greedy(const int* draft, const int* target, int batch, int nb,
                                int* accept, int* bonus, int* emitted, hipStream_t stream);
// ctx_lens[b] += accept[b], anchors[b] = bonus[b]; inj_seq / inj_pos [batch * nb] get the
// request index and the positions old ctx_lens[b] + j (clamped to max_ctx - 1).
hipError_t launch_advance(const int* accept, const int* bonus, int batch, int nb, int max_ctx,
                          int* ctx_lens, int* anchors, int* inj_seq, int* inj_pos,
                          hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace dflash
