// Launch interface of the block attention kernel.
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

constexpr int kAttnMaxChunks = 256;       // context chunks per (request, KV group)
constexpr int kAttnMaxChunkKeys = 4096;   // keys per chunk (256 pages)
constexpr int kAttnPidRegs = kAttnMaxChunkKeys / 16 / 64;   // page ids per lane of a chunk

// Query rows come in tiles of 16; request b owns rows b*rpr .. b*rpr + rpr - 1 (rpr / 16
// tiles) and rpr block keys, of which the first nbk are valid (causal: row j of the
// request's block also sees only block keys 0..j).
struct AttnArgs {
  const float* q;          // [B*rpr][n_q][d], RoPE applied
  const float* bk;         // [B][n_kv][rpr][d], block keys (RoPE applied)
  const float* bv;         // [B][n_kv][d][rpr], block values, transposed
  const void* k_pool;      // this layer's K pool [num_pages][n_kv][16][d]
  const void* v_pool;      // this layer's V pool [num_pages][n_kv][d][16]
  const int* block_table;  // page-table row of request b at block_table + b * table_ld
  int table_ld;            // max_pages, or 0 when every request reads one row
  int max_pages;
  const int* ctx_lens;     // [B]
  int rpr;                 // 16 or 32
  int nbk;                 // valid block keys, 1..rpr
  int causal;              // 1: block row j sees block keys 0..j only
  int n_q, n_kv, head_dim;
  int nc;                  // context chunks per request
  int chunk;               // context keys per chunk, a multiple of 32 (nc * chunk >= T_b)
  float scale;             // 1 / sqrt(d)
  float* part_o;           // [tiles][n_kv][nc][G][d/16][4][16 rows][4]
  float* part_ml;          // [tiles][n_kv][nc][G][16 rows][2]
  void* out;               // [B*rpr][n_q*d]: pair fragment layout (hilo_off) when out_hilo,
                           // else fp32 fragment layout (swz_off, kPer 4)
  int out_hilo;            // 1 for bf16 models, 0 for fp32 models
};

// tiles = B * rpr / 16.
hipError_t launch_block_attention(int bf16_dtype, const AttnArgs& a, int tiles,
                                  hipStream_t stream);
bool block_attention_supported(int bf16_dtype, int head_dim, int group);

}  // namespace dflash
