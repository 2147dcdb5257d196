// Host/device interface of the weight-streaming GEMM with fused epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

// Packed weight layout ("MFMA tile layout").  A weight W[N][K] is cut into tiles of 16 rows
// by kTile columns (kTile = 32 for bf16, 16 for fp32).  Tile (nt, kt) is 1024 contiguous
// bytes: lane l (0..63) owns 16 bytes holding W[16*nt + l%16][kTile*kt + kPerLane*(l/16) + j]
// for j < kPerLane.  Tiles are stored nt-major: byte offset (nt * KT + kt) * 1024 with
// KT = K / kTile.  One wave streaming one n-tile therefore reads contiguous 1 KB blocks,
// and each 16-byte lane chunk is directly the B operand of one MFMA step.
constexpr int kTileBytes = 1024;

enum Epi : int {
  EPI_STORE = 0,     // out[m][n] = acc, fp32 (fusion output c)
  EPI_RESIDUAL = 1,  // x[m][n] += acc, fp32 residual stream
  EPI_SWIGLU = 2,    // group = (gate tile, up tile): h[m][16*grp + c] = silu(gate) * up
  EPI_QKV = 3,       // group = one head of the fused Q|K|V projection: RoPE + scatter
  EPI_INJECT = 4,    // group = one K or V head of a layer: RoPE + paged-cache write
  EPI_ARGMAX = 5,    // LM head: running argmax per row, final ids by the last workgroup
};

struct GemmParams {
  // Operands
  const char* W;            // packed weights of grid.z slice 0
  long long w_zstride;      // bytes between grid.z slices
  int nt0;                  // first n-tile of this launch inside the packed matrix
  int KT;                   // k-tiles per n-tile row of the packed matrix
  const void* A;            // activations, row-major [M][lda]: fp32, or bf16 target features
  int lda;
  int M;                    // valid rows
  int n_tiles;              // n-tiles computed per grid.z slice
  int group;                // n-tiles per epilogue group
  int tpw;                  // n-tiles per workgroup (divides group; 1, 2 or 4)
  int splits;               // k-splits
  int kts;                  // k-tiles per split
  int n_mblocks;            // grid.y
  float* partials;          // split-K partial tiles (when a group spans >1 workgroup)
  unsigned* counters;       // one per (z, group, m-block); zero on entry and on exit

  // Epilogue operands
  void* out;                // EPI_STORE: [M][ldo] fp32 c; EPI_RESIDUAL: fp32 x;
                            // EPI_SWIGLU: [M][ldo] fp32 h
  int ldo;
  // EPI_QKV
  float* q_out;             // [M][n_q][d]
  float* bk_out;            // [M][n_kv][d]
  float* bv_out;            // [M][n_kv][d]
  const int* ctx_lens;      // [batch]; slot j of request b sits at ctx_lens[b] + j
  int n_q, n_kv, head_dim;
  double log_theta;
  // EPI_INJECT
  void* k_pool;
  void* v_pool;
  long long pool_layer_elems;  // elements per layer of a pool
  const int* block_table;
  int max_pages;
  const int* seq_idx;
  const int* pos;
  // EPI_ARGMAX
  unsigned long long* keys; // [M] running (value, index) keys, stride 16 words; zero on entry/exit
  int* ids_out;             // [M]
  float* logits_out;        // [M][ldo] or null
  unsigned* done_counter;   // launch-wide counter; zero on entry and exit
  int total_wgs;
};

// dtype_bf16: weight type; a_bf16: activation type of A (bf16 only for the fusion GEMM over
// the target features; otherwise fp32).
hipError_t launch_gemm(int dtype_bf16, int a_bf16, int mt, int epi, const GemmParams& p,
                       int layers, hipStream_t stream);

}  // namespace dflash
