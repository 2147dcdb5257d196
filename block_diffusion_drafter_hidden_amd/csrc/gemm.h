// Host/device interface of the weight-streaming GEMM with fused epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

// Packed weight layout ("MFMA tile layout").  A weight W[N][K] is cut into tiles of 16 rows
// by kTile columns (kTile = 32 for bf16, 16 for fp32).  Tile (nt, kt) is 1024 contiguous
// bytes: lane l (0..63) owns 16 bytes holding W[row(nt, l%16)][kTile*kt + kPerLane*(l/16) + j]
// for j < kPerLane.  Tiles are stored nt-major: byte offset (nt * KT + kt) * 1024 with
// KT = K / kTile.  One wave streaming one n-tile reads contiguous 1 KB blocks, and each
// 16-byte lane chunk is directly the B operand of one MFMA step.
//
// row(nt, r) is the identity except where an epilogue needs two rows side by side:
//   * RoPE heads (Q and K): tile t of a head holds dims i = 8t + r/2 (r even) and
//     i + d/2 (r odd), so each rotation pair sits in two adjacent columns of one tile;
//   * gate/up: tile j holds gate rows 8j..8j+7 (r < 8) and up rows 8j..8j+7 (r >= 8).
constexpr int kTileBytes = 1024;
constexpr int kMaxGemmThreads = 512;   // workgroup bound (ksub * tgpw <= 8 waves)

enum Epi : int {
  EPI_STORE = 0,     // out[m][n] = acc, fp32 (fusion output c)
  EPI_RESIDUAL = 1,  // x[m][n] += acc, fp32 residual stream
  EPI_SWIGLU = 2,    // tile j: h[m][8j + c] = silu(gate) * up, c < 8
  EPI_QKV = 3,       // fused Q|K|V projection: RoPE on Q/K pairs, scatter to q / block k, v
  EPI_INJECT = 4,    // one layer's K|V projection: RoPE on K pairs, write the paged cache
  EPI_ARGMAX = 5,    // LM head: per-row (value, index) maximum of each column block
};

// Where the activations (A) come from.
enum AKind : int {
  A_SWZ = 0,       // fp32 in the fragment layout (fp32 models; the fused feature c, which
                   // the injection splits into three bf16 pieces)
  A_ROW_F32 = 1,   // fp32 row-major [M][lda] (hidden rows handed in by a caller)
  A_ROW_BF16 = 2,  // bf16 row-major [M][lda] (target features of the fusion GEMM)
  A_HILO = 3,      // bf16 model activations as hi/lo pieces in the pair fragment layout
};

struct GemmParams {
  // Operands
  const char* W;            // packed weights of grid.z slice 0
  long long w_zstride;      // bytes between grid.z slices
  int nt0;                  // first n-tile of this launch inside the packed matrix
  int KT;                   // k-tiles per n-tile row of the packed matrix
  long long nt_stride;      // tiles between consecutive n-tiles (KT for the n-tile-major packing)
  long long kt_stride;      // tiles between consecutive k-tiles (1 for the n-tile-major packing)
  const void* A;            // activations (AKind)
  int lda;                  // row stride of the row-major kinds
  int M;                    // valid rows
  int a_kind;               // AKind
  // RMSNorm of the A rows (norm = 1).  The producer of A already multiplied it by the gain
  // and left the rows' sums of squares as `ssq_parts` partials, ssq_in[p * ssq_ld + row];
  // the kernel scales each finished row by 1 / sqrt(sum / K + eps).
  int norm;
  const float* ssq_in;
  int ssq_parts;
  int ssq_ld;               // row stride of the ssq arrays (padded rows)
  float eps;
  int n_tiles;              // n-tiles computed per grid.z slice
  int ksub;                 // waves splitting the k range of one tile group
  int kinter;               // 1: wave ks takes k-tiles ks, ks+ksub, ...; 0: a contiguous range
  int tgpw;                 // tile groups per workgroup (waves per workgroup = ksub * tgpw)
  int n_mblocks;            // grid.y

  // Epilogue operands
  void* out;                // EPI_STORE: c, EPI_RESIDUAL: x (fp32 fragment layout);
                            // EPI_SWIGLU: h (pair fragment layout for bf16 models, fp32
                            // fragment layout for fp32 models); ldo columns
  int ldo;
  // EPI_RESIDUAL, when xg_out is set: also write xg = x * gamma_next (as h) and the rows'
  // partial sums of squares ssq_out[part * ssq_ld + row] -- the inputs of the next
  // RMSNorm-folded GEMM.  Parts: one per n-tile (streaming kernel), one per 128-column block
  // (128-row kernel), or one per 512-column segment (128-row kernel with a k-split).
  void* xg_out;
  const float* gamma_next;
  float* ssq_out;
  // EPI_QKV
  float* q_out;             // [M][n_q][d]
  float* bk_out;            // [batch][n_kv][rpr slots][d]
  float* bv_out;            // [batch][n_kv][d][rpr slots] (transposed)
  const int* ctx_lens;      // [batch]; row j of request b (rows b*rpr ..) sits at ctx_lens[b] + j
  int rpr;                  // rows per request: 16 or 32
  int n_q, n_kv, head_dim;
  double inv_freq[64];      // RoPE frequencies theta^(-2i/d), i < d/2 (d <= 128)
  // EPI_INJECT, and EPI_QKV when k_pool is set (the input-fusion prefill): K/V of rows
  // m < kv_rows are also written to the paged cache (EPI_QKV: at its position, page
  // block_table[position / 16] of one request's table row; the block K/V then hold the
  // stored values).
  void* k_pool;
  void* v_pool;
  long long pool_layer_elems;  // elements per layer of a pool
  const int* block_table;
  int max_pages;
  const int* seq_idx;
  const int* pos;
  int kv_rows;
  // EPI_ARGMAX
  // (value, index) keys of each workgroup's best column per row, keys[part * keys_ld + row],
  // part = the workgroup's column block; reduced over parts by the finalize kernel.
  unsigned long long* keys;
  unsigned long long* keys2;   // may be null: the runner-up key of each part and row, same layout
  unsigned long long* keys3;   // refine mode: the third key of each part and row
  int keys_ld;
  float* logits_out;        // [rows][ldo] or null
  int draft_rpr;            // 0: plain rows; else rows are blocks of draft_rpr rows, and
  int draft_nb;             // slot j in 1..draft_nb-1 of block b is logits row b*(nb-1) + j-1
  // 256-row LM head only: multiply the hi piece of the input alone and leave each column
  // block's best three keys of those values for launch_argmax_refine, row-major:
  // keys[row * keys_ld + part] (keys_ld = the number of parts), likewise keys2, keys3.
  int refine;
  // 128-row kernel with EPI_RESIDUAL, EPI_STORE or EPI_QKV: the k range is split over
  // `ksplit` workgroups per output block (grid.y) and a reduction kernel adds the slices in
  // slice order and applies the epilogue.  Store / residual: slice s writes its fp32 partial
  // to partial[s][row][col] (M rows, ldo columns).  Q|K|V: slice s writes its un-normalized
  // 128 x 128 block b (row block major) to partial[(s * blocks + b) * 16384 + r * 128 + c].
  // ksplit <= 1: no split.
  int ksplit;
  float* partial;
  // bf16 feature rows with EPI_STORE: 256-row blocks (gemm_rows256), always through the
  // k-slice partials and their reduction (ksplit >= 1).
  int rows256;
};

// dtype_bf16: weight type; npw: n-tiles per wave (1, 2 or 4); the A kind and RMSNorm come
// from p.a_kind / p.norm.
hipError_t launch_gemm(int dtype_bf16, int mt, int npw, int epi, const GemmParams& p,
                       int layers, hipStream_t stream);

// ids[m] = index of the largest key over parts, keys[part * keys_ld + m], for m < rows; with
// draft_rpr the rows are blocks of draft_rpr rows and only slots 1..draft_nb-1 produce ids
// (block b, slot j -> ids[b*(draft_nb-1) + j-1]).  With keys2 (the parts' runner-up keys)
// and gap non-null, gap gets the difference of the best and second-best values of the row,
// same indexing as ids.
hipError_t launch_argmax_finalize(const unsigned long long* keys,
                                  const unsigned long long* keys2, int parts, int keys_ld,
                                  int* ids, float* gap, int rows, int draft_rpr, int draft_nb,
                                  hipStream_t stream);

// Exact argmax and top-2 gap of LM-head rows from a refine-mode launch (hi piece only).
// The bf16 input row is y = (hi + lo) * rstd; the hi-only value of a column differs from its
// exact value by at most rstd * |lo| * wmax (wmax: the largest LM-head row norm), so every
// column that can be among a row's top two has a hi value within twice that (plus a
// bound on both fp32 sums' rounding) of the second-best hi value.  Those columns -- each
// part's best three, or the whole part when its third-best is within the bound -- are
// recomputed exactly from the packed weights.  ids / gap / draft rows as for
// launch_argmax_finalize.
struct RefineArgs {
  const unsigned long long* keys;    // [rows][keys_ld] best hi-value key per row and part
  const unsigned long long* keys2;   // second keys, same layout
  const unsigned long long* keys3;   // third keys, same layout
  int parts, keys_ld, part_cols;
  const void* a;                     // LM-head input rows, pair fragment layout (bf16 pieces)
  int KT;                            // k-tiles of 32 (hidden / 32)
  const float* ssq;                  // partial sums of squares of the rows (as the GEMM's)
  int ssq_parts, ssq_ld;
  float eps;
  const char* w;                     // packed LM head
  long long nt_stride, kt_stride;
  int vocab;
  const float* wmax;                 // largest LM-head row norm (device)
  int* ids;
  float* gap;
  int draft_rpr, draft_nb;
};
constexpr int kRefineMaxHidden = 8192;
hipError_t launch_argmax_refine(const RefineArgs& a, int rows, hipStream_t stream);

// Column blocks (argmax parts) of an EPI_ARGMAX launch with this plan.
inline int argmax_parts(int n_tiles, int mt, int npw, int tgpw) {
  return mt == 8 ? (n_tiles + 7) / 8 : n_tiles / (npw * tgpw);
}

}  // namespace dflash
