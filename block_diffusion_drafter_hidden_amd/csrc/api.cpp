// Host side of the DFlash C ABI: argument validation, packed-weight and workspace layouts,
// GEMM planning, and the launch sequence of each step call.  Nothing here allocates device
// memory or synchronizes; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "dflash.h"
#include "attention.h"
#include "common.h"
#include "gemm.h"
#include "sampled.h"
#include "small.h"

using namespace dflash;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kSyncBytes = kAlign;                  // reserved head of a workspace
constexpr int kMaxBatch = 4096;                         // requests per draft call
constexpr int kMaxPagesPerSeq = 16384;   // 262144 positions per request
static_assert(kMaxPagesPerSeq * 16 <= kAttnMaxChunks * kAttnMaxChunkKeys,
              "the attention's chunks cover the longest context");
// Waves a streaming-GEMM plan aims at: with the load ring, 4 k-slices per tile group ran the
// one-request Q|K|V, O, down and fusion GEMMs 1-10% faster than 8 (same box).
constexpr int kTargetWaves = 768;
constexpr int kAttnTargetWGs = 128;   // context-chunk workgroups wanted at small batch

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

struct Dims {
  int L, H, nq, nkv, d, I, V, F, G;
  int bf16;
  size_t es;   // element size of weights / operands
  int ktile;   // K per k-tile
  float theta, eps;
  int mask;
  int nb;      // block size: 8, 16 or 32
  int rpr;     // rows per request of a draft pass: max(nb, 16)
};

dflash_status check_config(const dflash_config* c, Dims* o) {
  if (!c) return DFLASH_ERR_INVALID_ARG;
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0 || c->feat_dim <= 0)
    return DFLASH_ERR_INVALID_ARG;
  if ((c->block_size != 8 && c->block_size != 16 && c->block_size != 32) || c->page_size != 16)
    return DFLASH_ERR_UNSUPPORTED;
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_ERR_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads) return DFLASH_ERR_INVALID_ARG;
  if (c->hidden % 64 || c->feat_dim % 64 || c->intermediate % 64 || c->vocab % 64)
    return DFLASH_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (!block_attention_supported(c->dtype == DFLASH_BF16, c->head_dim,
                                 c->n_q_heads / c->n_kv_heads))
    return DFLASH_ERR_UNSUPPORTED;
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return DFLASH_ERR_INVALID_ARG;
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return DFLASH_ERR_INVALID_ARG;
  if (o) {
    o->L = c->n_layers;
    o->H = c->hidden;
    o->nq = c->n_q_heads;
    o->nkv = c->n_kv_heads;
    o->d = c->head_dim;
    o->I = c->intermediate;
    o->V = c->vocab;
    o->F = c->feat_dim;
    o->G = c->n_q_heads / c->n_kv_heads;
    o->bf16 = c->dtype == DFLASH_BF16;
    o->es = o->bf16 ? 2 : 4;
    o->ktile = o->bf16 ? 32 : 16;
    o->theta = c->rope_theta;
    o->eps = c->rms_eps;
    o->mask = c->mask_token_id;
    o->nb = c->block_size;
    o->rpr = std::max(c->block_size, kQRows);
  }
  return DFLASH_OK;
}

// ---------------------------------------------------------------------------------------
// Packed weight buffer layout.
// ---------------------------------------------------------------------------------------
struct Packed {
  size_t final_norm, w_fuse, lm_head, lm_norms, lm_wmax, layer0, layer_stride;
  size_t attn_norm, mlp_norm, wqkv, wo, wgu, wd;  // offsets inside one layer
  size_t total;
};

Packed packed_layout(const Dims& m) {
  Packed p{};
  size_t off = 0;
  p.final_norm = off;
  off = align_up(off + (size_t)m.H * 4);
  p.w_fuse = off;
  off = align_up(off + (size_t)m.H * m.F * m.es);
  p.lm_head = off;
  off = align_up(off + (size_t)m.V * m.H * m.es);
  p.lm_norms = off;   // the LM head's row norms, then the largest of them
  off = align_up(off + (size_t)m.V * 4);
  p.lm_wmax = off;
  off = align_up(off + 4);
  p.layer0 = off;
  size_t lo = 0;
  p.attn_norm = lo;
  lo = align_up(lo + (size_t)m.H * 4);
  p.mlp_norm = lo;
  lo = align_up(lo + (size_t)m.H * 4);
  p.wqkv = lo;
  lo = align_up(lo + (size_t)(m.nq + 2 * m.nkv) * m.d * m.H * m.es);
  p.wo = lo;
  lo = align_up(lo + (size_t)m.H * m.nq * m.d * m.es);
  p.wgu = lo;
  lo = align_up(lo + (size_t)2 * m.I * m.H * m.es);
  p.wd = lo;
  lo = align_up(lo + (size_t)m.H * m.I * m.es);
  p.layer_stride = lo;
  p.total = off + lo * m.L;
  return p;
}

// ---------------------------------------------------------------------------------------
// GEMM planning.  Waves split the k range of a tile group (ksub), a workgroup holds tgpw tile
// groups; the plan aims at >= kTargetWaves waves in flight with >= 8 k-tiles per wave.
// (Sweeps over the batch-1 shapes on MI355X: the LM head prefers 2 waves per k range and 2
// tile groups of 4 n-tiles; the other GEMMs 4 waves per k range.)
// ---------------------------------------------------------------------------------------
struct Plan {
  int mt, n_mblocks, npw, ksub, tgpw;
  bool rows256;   // the fusion over 256-row blocks (gemm_rows256), always through partials
};

// Rows above which bf16 GEMMs use the 128 x 128 tall kernel (weights read once per 128 rows
// instead of once per 64; a ragged last column block is allowed).
constexpr int kTallRows = 64;
constexpr int kTallMT = 8;
constexpr int kTallNT = 8;   // n-tiles per 128-column block of the 128-row kernel

Plan plan_gemm(int n_tiles, int KT, int M, int npw, int layers, int max_ksub = 16,
               bool tall_ok = false) {
  Plan p{};
  if (tall_ok && M > kTallRows) {
    p.mt = kTallMT;
    p.n_mblocks = cdiv(M, 16 * kTallMT);
    p.npw = 1;
    p.ksub = 1;
    p.tgpw = 1;
    return p;
  }
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.n_mblocks = cdiv(std::max(M, 1), 16 * p.mt);
  p.npw = npw;
  const int groups = n_tiles / npw;
  const long long units = (long long)groups * p.n_mblocks * layers;
  const int max_waves = std::max(1, std::min(kMaxGemmThreads / 64, 16 / (npw * p.mt)));
  auto tile_fits = [&](int tg) { return p.mt * 16 * (tg * npw * 16 + 1) <= 64 * 65; };
  p.ksub = 1;
  while (p.ksub < max_ksub && units * p.ksub < kTargetWaves && KT / (p.ksub * 2) >= 8 &&
         p.ksub * 2 <= max_waves)
    p.ksub *= 2;
  p.tgpw = 1;
  // A wide GEMM whose tile groups split evenly over 256 workgroups runs one workgroup per CU
  // with t tile groups each (t need not be a power of two).
  const long long wgs1 = (long long)groups * p.n_mblocks * layers;
  if (wgs1 >= 512 && wgs1 % 256 == 0 && groups % (wgs1 / 256) == 0) {
    const int t = (int)(wgs1 / 256);
    if (t <= max_waves && tile_fits(t)) {
      p.tgpw = t;
      p.ksub = 1;
      while (p.ksub * 2 * t <= max_waves && KT / (p.ksub * 2) >= 8) p.ksub *= 2;
      return p;
    }
  }
  while (p.ksub * p.tgpw < 4 && p.ksub * p.tgpw * 2 <= max_waves &&
         groups % (p.tgpw * 2) == 0 && tile_fits(p.tgpw * 2))
    p.tgpw *= 2;
  return p;
}

// Partial sums of squares per row that a residual GEMM with this plan leaves for the next
// norm: one per n-tile (streaming kernel), one per 128-column block (128-row kernel), one
// per 512-column segment (128-row kernel with a k-split: the segments of its reduction
// kernel).
int residual_ssq_parts(const Plan& pl, int n_tiles) {
  if (pl.mt != kTallMT) return n_tiles;
  return pl.ksub > 1 ? cdiv(n_tiles, 32) : cdiv(n_tiles, kTallNT);
}

// RoPE frequencies theta^(-2i/d) in fp64 for the epilogues that rotate q and k.
void set_rope(const Dims& m, GemmParams& g) {
  const double log_theta = std::log((double)m.theta);
  for (int i = 0; i < m.d / 2; ++i) g.inv_freq[i] = std::exp(-(2.0 * i / m.d) * log_theta);
}

// How the drafter's own activations are stored: bf16 models keep them as ready-made hi/lo
// bf16 pieces (pair fragment layout), fp32 models as fp32 fragments.
int act_kind(const Dims& m) { return m.bf16 ? A_HILO : A_SWZ; }

GemmParams base_params(const Plan& pl, const char* W, int nt0, int KT, const void* A, int lda,
                       int M, int n_tiles) {
  GemmParams g;
  std::memset(&g, 0, sizeof(g));
  g.W = W;
  g.nt0 = nt0;
  g.KT = KT;
  g.nt_stride = KT;
  g.kt_stride = 1;
  g.A = A;
  g.lda = lda;
  g.M = M;
  g.a_kind = A_SWZ;
  g.norm = 0;
  g.n_tiles = n_tiles;
  g.ksub = pl.ksub;
  g.tgpw = pl.tgpw;
  g.n_mblocks = pl.n_mblocks;
  return g;
}

struct Carver {
  size_t off;
  explicit Carver(size_t start) : off(start) {}
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// The LM head's plan (the streaming kernel prefers 2 waves per k range and 2 tile groups of
// 4 n-tiles at one m-tile) and the bytes of its argmax partials.
Plan lm_plan(const Dims& m, int rows) {
  // 4 n-tiles per wave up to two m-tiles; at four m-tiles two (4 x 4 tiles of two
  // accumulator chains and the load ring would not fit the register file).
  const int mt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  Plan pl = plan_gemm(m.V / 16, m.H / m.ktile, rows, mt == 4 ? 2 : 4, 1, 16, m.bf16 != 0);
  if (pl.mt == 1 && (m.V / 16 / 4) % 2 == 0 && m.H / m.ktile >= 32) {
    pl.ksub = 2;
    pl.tgpw = 2;
  }
  return pl;
}
// Best and runner-up keys per (part, row): two arrays of this many bytes each.
size_t lm_keys_bytes(const Dims& m, int rows) {
  const Plan pl = lm_plan(m, rows);
  return (size_t)argmax_parts(m.V / 16, pl.mt, pl.npw, pl.tgpw) * rows * 8;
}

// ---------------------------------------------------------------------------------------
// Per-call plans of the draft and inject steps.
// ---------------------------------------------------------------------------------------
struct DraftPlan {
  Plan qkv, o, gu, dn;
  int nc, chunk;
  size_t x, xg, ssq, q, bk, bv, ao, h, apart_o, apart_ml, keys, kpart;
  size_t total;
};

// k-slices of a 128-row store, residual or Q|K|V GEMM: at least `min_wgs` workgroups (up to
// max_s slices) and at least 32 k-tiles per slice.  Measured: Q|K|V wants one workgroup per
// CU (256), the residual GEMMs two rounds but at most two slices, the deep-K fusion 512.
int ksplit_count(const Plan& pl, int n_tiles, int KT, int min_wgs, int max_s = 8) {
  if (pl.mt != kTallMT) return 1;
  const long long blocks = (long long)cdiv(n_tiles, 8) * pl.n_mblocks;
  int s = 1;
  while (blocks * s < min_wgs && KT / (s * 2) >= 32 && s < max_s) s *= 2;
  return s;
}

DraftPlan draft_plan(const Dims& m, int B, int max_ctx) {
  DraftPlan p{};
  const int rows = B * m.rpr;
  const int tiles = rows / kQRows;
  const bool tall = m.bf16 != 0;
  p.qkv = plan_gemm((m.nq + 2 * m.nkv) * m.d / 16, m.H / m.ktile, rows, 2, 1, 16, tall);
  p.o = plan_gemm(m.H / 16, m.nq * m.d / m.ktile, rows, 1, 1, 16, tall);
  p.gu = plan_gemm(2 * m.I / 16, m.H / m.ktile, rows, 2, 1, 16, tall);
  p.dn = plan_gemm(m.H / 16, m.I / m.ktile, rows, 1, 1, 16, tall);
  const int qkv_tiles = (m.nq + 2 * m.nkv) * m.d / 16;
  if (p.qkv.mt == kTallMT) p.qkv.ksub = ksplit_count(p.qkv, qkv_tiles, m.H / m.ktile, 256);
  // O and down: two rounds of workgroups (512), but at most two k-slices (same box: LLaMA
  // batch 64 7.27 -> 7.16 ms, gpt-oss batch 128 22.37 -> 21.99 ms per step; four slices at
  // 512 rows were slower than two).
  if (p.o.mt == kTallMT) p.o.ksub = ksplit_count(p.o, m.H / 16, m.nq * m.d / m.ktile, 512, 2);
  if (p.dn.mt == kTallMT) p.dn.ksub = ksplit_count(p.dn, m.H / 16, m.I / m.ktile, 512, 2);
  const int kv_groups = tiles * m.nkv;
  const int max_chunks = std::max(1, cdiv(std::max(max_ctx, 1), 32));
  // Context chunks per (request, KV group): enough workgroups to fill the chip at small
  // batch; otherwise the longest chunks the kernel takes (4096 keys), which minimize the
  // partials written and merged (measured faster than ~512-key chunks at batch 16-64).
  const int want = std::max(cdiv(kAttnTargetWGs, kv_groups),
                            cdiv(std::max(max_ctx, 1), kAttnMaxChunkKeys));
  p.nc = std::max(1, std::min({want, max_chunks, kAttnMaxChunks}));
  p.chunk = cdiv(cdiv(std::max(max_ctx, 1), p.nc), 32) * 32;
  Carver c(kSyncBytes);
  p.x = c.take((size_t)rows * m.H * 4);
  p.xg = c.take((size_t)rows * m.H * 4);
  p.ssq = c.take((size_t)(m.H / 16) * rows * 4);
  p.q = c.take((size_t)rows * m.nq * m.d * 4);
  p.bk = c.take((size_t)rows * m.nkv * m.d * 4);
  p.bv = c.take((size_t)rows * m.nkv * m.d * 4);
  p.ao = c.take((size_t)rows * m.nq * m.d * 4);
  p.h = c.take((size_t)rows * m.I * 4);
  const size_t R = (size_t)m.G * 16;
  p.apart_o = c.take((size_t)kv_groups * p.nc * R * m.d * 4);
  p.apart_ml = c.take((size_t)kv_groups * p.nc * R * 2 * 4);
  p.keys = c.take(3 * lm_keys_bytes(m, rows));
  // k-split partials: row-major for the O and down projections, whole 128 x 128 blocks for
  // Q|K|V (one buffer, used by one GEMM at a time).
  const int splits = std::max(p.o.mt == kTallMT ? p.o.ksub : 1, p.dn.mt == kTallMT ? p.dn.ksub : 1);
  const size_t row_part = splits > 1 ? (size_t)splits * rows * m.H * 4 : 0;
  const int qkv_splits = p.qkv.mt == kTallMT ? p.qkv.ksub : 1;
  const size_t tile_part = qkv_splits > 1 ? (size_t)qkv_splits * cdiv(qkv_tiles, 8) *
                                                p.qkv.n_mblocks * kTallMT * 16 * 128 * 4
                                          : 0;
  p.kpart = c.take(std::max(row_part, tile_part));
  p.total = c.off;
  return p;
}

struct InjectPlan {
  Plan fuse, kv;
  size_t c, fpart, total;
};

// The fusion GEMM (narrow N = H, deep K = F) splits K: over waves at few rows, over
// workgroups in the 128-row kernel, and from 256 bf16 rows on it runs over 256-row blocks
// (gemm_rows256) with the k-slices that give 512 workgroups.
Plan fuse_plan(const Dims& m, int rows) {
  Plan pl = plan_gemm(m.H / 16, m.F / m.ktile, rows, 1, 1, 16, m.bf16 != 0);
  if (pl.mt != kTallMT) return pl;
  const int KT = m.F / m.ktile;
  if (rows >= 256) {
    pl.rows256 = true;
    const long long blocks = (long long)cdiv(m.H / 16, 8) * cdiv(rows, 256);
    int s = 1;
    while (blocks * s < 512 && KT / (s * 2) >= 32 && s < 8) s *= 2;
    pl.ksub = s;
    return pl;
  }
  pl.ksub = ksplit_count(pl, m.H / 16, KT, 512);
  return pl;
}
// Bytes of the fusion's k-slice partials.
size_t fuse_partial_bytes(const Dims& m, const Plan& pl, int rows) {
  const int splits = pl.mt == kTallMT ? pl.ksub : 1;
  return splits > 1 || pl.rows256 ? (size_t)splits * rows * m.H * 4 : 0;
}

InjectPlan inject_plan(const Dims& m, int rows) {
  InjectPlan p{};
  p.fuse = fuse_plan(m, rows);
  p.kv = plan_gemm(2 * m.nkv * m.d / 16, m.H / m.ktile, rows, 2, m.L, 4, m.bf16 != 0);
  Carver c(kSyncBytes);
  p.c = c.take((size_t)cdiv(rows, 16) * 16 * m.H * 4);   // fragment layout: rows padded
  p.fpart = c.take(fuse_partial_bytes(m, p.fuse, rows));
  p.total = c.off;
  return p;
}

constexpr int kInjectChunkRows = 1024;   // rows per fusion + injection launch pair, at most

// The input-fusion prefill: context rows pass through the layers in chunks of at most
// kPrefillChunkRows rows, each chunk as kPrefillChunkRows / 16 groups of 16 rows that the
// draft pass's kernels take as "requests" (rows padded to a multiple of 16).
constexpr int kPrefillChunkRows = 2048;

struct PrefillPlan {
  DraftPlan dp;     // layer buffers for rows / 16 groups of 16 rows
  size_t fpart;     // k-split partials of the fusion GEMM (the largest any chunk needs)
  size_t gctx;      // [groups] cached context of each group
  size_t total;
};

// The layer plan of a prefill chunk of `groups` 16-row groups.
DraftPlan prefill_layer_plan(const Dims& m, int groups, int max_ctx) {
  Dims g = m;
  g.rpr = kQRows;   // one 16-row group per "request"
  g.nb = kQRows;
  return draft_plan(g, groups, max_ctx);
}

Plan prefill_fuse_plan(const Dims& m, int rows) { return fuse_plan(m, rows); }

// rows: padded rows of the largest chunk (a multiple of 16, at most kPrefillChunkRows).
PrefillPlan prefill_plan(const Dims& m, int rows, int max_ctx) {
  PrefillPlan p{};
  p.dp = prefill_layer_plan(m, rows / kQRows, max_ctx);
  // A shorter (last) chunk can take more k-slices than a full one: the layer buffers and
  // the fusion partials are sized for the largest need of any chunk length.
  size_t layers = p.dp.total, part = 0;
  for (int r = 16; r <= rows; r += 16) {
    layers = std::max(layers, prefill_layer_plan(m, r / kQRows, max_ctx).total);
    part = std::max(part, fuse_partial_bytes(m, prefill_fuse_plan(m, r), r));
  }
  Carver c(layers);
  p.fpart = c.take(part);
  p.gctx = c.take((size_t)(rows / kQRows) * 4);
  p.total = c.off;
  return p;
}

#define DF_TRY(expr)                                  \
  do {                                                \
    hipError_t _e = (expr);                           \
    if (_e != hipSuccess) return DFLASH_ERR_HIP;      \
  } while (0)

// Final RMSNorm + shared LM head + argmax over the vocabulary.  `xg` is x * final gain in
// the fragment layout and ssq the rows' sums of squares (ssq_parts partials, row stride
// ssq_ld); with draft_rows the rows are 16-slot blocks and slot 0 is computed and dropped.
// keys: workspace for the per-column-block argmax partials, 3 * lm_keys_bytes(m, rows)
// bytes (best keys, then runner-up keys, written when gap_out is set or in refine mode,
// then third keys, refine mode only).
// draft: the rows are draft blocks (m.rpr rows per request, ids of slots 1 .. m.nb - 1).
dflash_status launch_lm_head(const Dims& m, const Packed& P, const char* wb, const void* xg,
                             const float* ssq, int ssq_parts, int ssq_ld, int rows,
                             bool draft, int* ids_out, float* gap_out, float* logits_out,
                             unsigned long long* keys, hipStream_t stream) {
  const Plan pl = lm_plan(m, rows);
  const int parts = argmax_parts(m.V / 16, pl.mt, pl.npw, pl.tgpw);
  // Past 64 rows (the 256-row kernel, where the LM head is matrix-core bound) and without
  // logits to return: the hi piece alone, then the exact top two of the columns that can
  // still win (launch_argmax_refine) -- half the matrix-core work, the same ids and gaps.
  const bool refine = pl.mt == kTallMT && !logits_out && m.H <= kRefineMaxHidden &&
                      parts <= 2048;
  GemmParams g = base_params(pl, wb + P.lm_head, 0, m.H / m.ktile, xg, m.H, rows, m.V / 16);
  g.a_kind = act_kind(m);
  g.norm = 1;
  g.ssq_in = ssq;
  g.ssq_parts = ssq_parts;
  g.ssq_ld = ssq_ld;
  g.eps = m.eps;
  g.keys = keys;
  g.keys2 = (gap_out || refine) ? keys + lm_keys_bytes(m, rows) / 8 : nullptr;
  g.keys3 = refine ? keys + 2 * (lm_keys_bytes(m, rows) / 8) : nullptr;
  g.refine = refine ? 1 : 0;
  g.keys_ld = refine ? parts : rows;
  g.logits_out = logits_out;
  // The two waves of a k range take alternate k-tiles, so a workgroup reads its n-tiles'
  // weights front to back together (streaming kernel; LM-head launch 204.5 -> 202.5 us at one
  // request, same box; the other GEMMs measured slower this way).
  g.kinter = 1;
  g.ldo = m.V;
  g.draft_rpr = draft ? m.rpr : 0;
  g.draft_nb = m.nb;
  DF_TRY(launch_gemm(m.bf16, pl.mt, pl.npw, EPI_ARGMAX, g, 1, stream));
  if (refine) {
    RefineArgs r{};
    r.keys = keys;
    r.keys2 = g.keys2;
    r.keys3 = g.keys3;
    r.parts = parts;
    r.keys_ld = parts;
    r.part_cols = 16 * kTallNT;
    r.a = xg;
    r.KT = m.H / m.ktile;
    r.ssq = ssq;
    r.ssq_parts = ssq_parts;
    r.ssq_ld = ssq_ld;
    r.eps = m.eps;
    r.w = wb + P.lm_head;
    r.nt_stride = m.H / m.ktile;
    r.kt_stride = 1;
    r.vocab = m.V;
    r.wmax = reinterpret_cast<const float*>(wb + P.lm_wmax);
    r.ids = ids_out;
    r.gap = gap_out;
    r.draft_rpr = g.draft_rpr;
    r.draft_nb = g.draft_nb;
    DF_TRY(launch_argmax_refine(r, rows, stream));
    return DFLASH_OK;
  }
  DF_TRY(launch_argmax_finalize(keys, g.keys2, parts, rows, ids_out, gap_out, rows,
                                g.draft_rpr, g.draft_nb, stream));
  return DFLASH_OK;
}

}  // namespace

// =========================================================================================
// C ABI
// =========================================================================================
extern "C" {

const char* dflash_error_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_INVALID_ARG: return "invalid argument";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DFLASH_ERR_WORKSPACE: return "workspace or packed buffer too small";
    case DFLASH_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t dflash_packed_weights_size(const dflash_config* cfg) {
  Dims m;
  if (check_config(cfg, &m) != DFLASH_OK) return 0;
  return packed_layout(m).total;
}

dflash_status dflash_pack_weights(const dflash_config* cfg, const dflash_weights* w,
                                  void* packed, size_t packed_bytes, hipStream_t stream) {
  Dims m;
  dflash_status st = check_config(cfg, &m);
  if (st != DFLASH_OK) return st;
  if (!w || !packed || !w->w_fuse || !w->lm_head || !w->final_norm || !w->attn_norm ||
      !w->wq || !w->wk || !w->wv || !w->wo || !w->mlp_norm || !w->w_gate || !w->w_up ||
      !w->w_down)
    return DFLASH_ERR_INVALID_ARG;
  for (int l = 0; l < m.L; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] ||
        !w->mlp_norm[l] || !w->w_gate[l] || !w->w_up[l] || !w->w_down[l])
      return DFLASH_ERR_INVALID_ARG;
  const Packed P = packed_layout(m);
  if (packed_bytes < P.total) return DFLASH_ERR_WORKSPACE;
  char* base = reinterpret_cast<char*>(packed);

  auto pack1 = [&](const void* src, int N, int K, size_t off) -> hipError_t {
    PackArgs a{};
    a.src[0] = src;
    a.seg_tiles[0] = N / 16;
    a.n_segs = 1;
    a.mode = PACK_CONCAT;
    a.n_tiles_total = N / 16;
    a.KT = K / m.ktile;
    a.K = K;
    a.dst = base + off;
    return launch_pack(m.bf16, a, stream);
  };
  DF_TRY(launch_widen(m.bf16, w->final_norm, reinterpret_cast<float*>(base + P.final_norm), m.H,
                      stream));
  DF_TRY(pack1(w->w_fuse, m.H, m.F, P.w_fuse));
  DF_TRY(pack1(w->lm_head, m.V, m.H, P.lm_head));
  DF_TRY(launch_row_norm_max(m.bf16, w->lm_head, m.V, m.H,
                             reinterpret_cast<float*>(base + P.lm_norms),
                             reinterpret_cast<float*>(base + P.lm_wmax), stream));
  for (int l = 0; l < m.L; ++l) {
    const size_t lb = P.layer0 + (size_t)l * P.layer_stride;
    DF_TRY(launch_widen(m.bf16, w->attn_norm[l], reinterpret_cast<float*>(base + lb + P.attn_norm),
                        m.H, stream));
    DF_TRY(launch_widen(m.bf16, w->mlp_norm[l], reinterpret_cast<float*>(base + lb + P.mlp_norm),
                        m.H, stream));
    PackArgs q{};
    q.src[0] = w->wq[l];
    q.src[1] = w->wk[l];
    q.src[2] = w->wv[l];
    q.seg_tiles[0] = m.nq * m.d / 16;
    q.seg_tiles[1] = m.nkv * m.d / 16;
    q.seg_tiles[2] = m.nkv * m.d / 16;
    q.n_segs = 3;
    q.mode = PACK_CONCAT;
    q.rope_segs = 2;   // Q and K heads: rotation pairs side by side
    q.head_dim = m.d;
    q.n_tiles_total = (m.nq + 2 * m.nkv) * m.d / 16;
    q.KT = m.H / m.ktile;
    q.K = m.H;
    q.dst = base + lb + P.wqkv;
    DF_TRY(launch_pack(m.bf16, q, stream));
    DF_TRY(pack1(w->wo[l], m.H, m.nq * m.d, lb + P.wo));
    PackArgs gu{};
    gu.src[0] = w->w_gate[l];
    gu.src[1] = w->w_up[l];
    gu.seg_tiles[0] = m.I / 16;
    gu.seg_tiles[1] = m.I / 16;
    gu.n_segs = 2;
    gu.mode = PACK_GATE_UP;
    gu.n_tiles_total = 2 * m.I / 16;
    gu.KT = m.H / m.ktile;
    gu.K = m.H;
    gu.dst = base + lb + P.wgu;
    DF_TRY(launch_pack(m.bf16, gu, stream));
    DF_TRY(pack1(w->w_down[l], m.H, m.I, lb + P.wd));
  }
  return DFLASH_OK;
}

size_t dflash_workspace_size(const dflash_config* cfg, int32_t max_batch,
                             int32_t max_inject_rows, int32_t max_ctx) {
  Dims m;
  if (check_config(cfg, &m) != DFLASH_OK) return 0;
  if (max_batch < 0 || max_inject_rows < 0 || max_ctx < 0) return 0;
  size_t need = kSyncBytes;
  if (max_batch > 0) need = std::max(need, draft_plan(m, max_batch, max_ctx).total);
  if (max_inject_rows > 0) {
    // every injection of up to max_inject_rows rows in one chunk (fewer rows can take more
    // k-slices of the fusion)
    const int R = std::min(max_inject_rows, kInjectChunkRows);
    for (int r = 16; r < R; r += 16) need = std::max(need, inject_plan(m, r).total);
    need = std::max(need, inject_plan(m, R).total);
  }
  return need;
}

dflash_status dflash_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!workspace) return DFLASH_ERR_INVALID_ARG;
  if (ws_bytes < kSyncBytes) return DFLASH_ERR_WORKSPACE;
  DF_TRY(launch_zero(workspace, kSyncBytes, stream));
  return DFLASH_OK;
}

static dflash_status check_cache(const dflash_kv_cache* c) {
  if (!c || !c->k_pool || !c->v_pool || !c->block_table || !c->ctx_lens) return DFLASH_ERR_INVALID_ARG;
  if (c->num_pages <= 0 || c->max_pages_per_seq <= 0) return DFLASH_ERR_INVALID_ARG;
  return DFLASH_OK;
}

dflash_status dflash_fuse_inject_kv(const dflash_config* cfg, const void* packed,
                                    const dflash_kv_cache* cache, const void* feats,
                                    const int32_t* seq_idx, const int32_t* pos, int32_t n_tok,
                                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  Dims m;
  dflash_status st = check_config(cfg, &m);
  if (st != DFLASH_OK) return st;
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  if (!packed || !workspace || n_tok < 0) return DFLASH_ERR_INVALID_ARG;
  if (n_tok == 0) return DFLASH_OK;
  if (!feats || !seq_idx || !pos) return DFLASH_ERR_INVALID_ARG;
  // The largest chunk (up to kInjectChunkRows rows) whose buffers fit the workspace.
  int chunk_rows = std::min<int>(n_tok, kInjectChunkRows);
  InjectPlan ip = inject_plan(m, chunk_rows);
  while (ip.total > ws_bytes && chunk_rows > 16) {
    chunk_rows = std::max(16, chunk_rows / 2);
    ip = inject_plan(m, chunk_rows);
  }
  if (ws_bytes < ip.total) return DFLASH_ERR_WORKSPACE;
  const Packed P = packed_layout(m);
  const char* wb = reinterpret_cast<const char*>(packed);
  char* ws = reinterpret_cast<char*>(workspace);
  float* cbuf = reinterpret_cast<float*>(ws + ip.c);
  const long long pool_layer = (long long)cache->num_pages * m.nkv * 16 * m.d;

  for (int r0 = 0; r0 < n_tok; r0 += chunk_rows) {
    const int rows = std::min(chunk_rows, n_tok - r0);
    InjectPlan cp = rows == chunk_rows ? ip : inject_plan(m, rows);
    // a short last chunk's extra k-slices: unsplit (its partial then needs rows x H floats,
    // within the first chunk's)
    if (cp.total > ws_bytes) cp.fuse.ksub = 1;
    {  // fusion of the concatenated target features: c = W_fuse . X (fp32 out)
      GemmParams g = base_params(cp.fuse, wb + P.w_fuse, 0, m.F / m.ktile,
                                 reinterpret_cast<const char*>(feats) + (size_t)r0 * m.F * m.es,
                                 m.F, rows, m.H / 16);
      g.a_kind = m.bf16 ? A_ROW_BF16 : A_ROW_F32;
      g.out = cbuf;
      g.ldo = m.H;
      g.ksplit = cp.fuse.mt == kTallMT ? cp.fuse.ksub : 1;
      g.rows256 = cp.fuse.rows256;
      g.partial = reinterpret_cast<float*>(ws + cp.fpart);
      DF_TRY(launch_gemm(m.bf16, cp.fuse.mt, cp.fuse.npw, EPI_STORE, g, 1, stream));
    }
    {  // every layer's K|V projection of c, RoPE on K, written into the paged cache
      GemmParams g = base_params(cp.kv, wb + P.layer0 + P.wqkv, m.nq * m.d / 16, m.H / m.ktile,
                                 cbuf, m.H, rows, 2 * m.nkv * m.d / 16);
      g.w_zstride = (long long)P.layer_stride;
      g.n_q = m.nq;
      g.n_kv = m.nkv;
      g.head_dim = m.d;
      set_rope(m, g);
      g.k_pool = cache->k_pool;
      g.v_pool = cache->v_pool;
      g.pool_layer_elems = pool_layer;
      g.block_table = cache->block_table;
      g.max_pages = cache->max_pages_per_seq;
      g.seq_idx = seq_idx + r0;
      g.pos = pos + r0;
      DF_TRY(launch_gemm(m.bf16, cp.kv.mt, cp.kv.npw, EPI_INJECT, g, m.L, stream));
    }
  }
  return DFLASH_OK;
}

size_t dflash_prefill_workspace_size(const dflash_config* cfg, int32_t max_tok,
                                     int32_t max_ctx) {
  Dims m;
  if (check_config(cfg, &m) != DFLASH_OK) return 0;
  if (max_tok < 0 || max_ctx < 0) return 0;
  const int rows = std::min(cdiv(std::max(max_tok, 1), 16) * 16, kPrefillChunkRows);
  return prefill_plan(m, rows, max_ctx).total;
}

dflash_status dflash_prefill_input_fusion(const dflash_config* cfg, const void* packed,
                                          const dflash_kv_cache* cache, const void* feats,
                                          int32_t seq, int32_t n_tok, void* workspace,
                                          size_t ws_bytes, hipStream_t stream) {
  Dims m;
  dflash_status st = check_config(cfg, &m);
  if (st != DFLASH_OK) return st;
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  if (!packed || !workspace || n_tok < 0 || seq < 0) return DFLASH_ERR_INVALID_ARG;
  if (n_tok == 0) return DFLASH_OK;
  if (!feats) return DFLASH_ERR_INVALID_ARG;
  if (cache->max_pages_per_seq > kMaxPagesPerSeq) return DFLASH_ERR_UNSUPPORTED;
  const int max_ctx = cache->max_pages_per_seq * 16;
  if (n_tok > max_ctx) return DFLASH_ERR_INVALID_ARG;
  const int chunk_rows = std::min(cdiv(n_tok, 16) * 16, kPrefillChunkRows);
  const PrefillPlan pp = prefill_plan(m, chunk_rows, max_ctx);
  if (ws_bytes < pp.total) return DFLASH_ERR_WORKSPACE;
  const DraftPlan& dp = pp.dp;

  const Packed P = packed_layout(m);
  const char* wb = reinterpret_cast<const char*>(packed);
  char* ws = reinterpret_cast<char*>(workspace);
  float* x = reinterpret_cast<float*>(ws + dp.x);
  float* xg = reinterpret_cast<float*>(ws + dp.xg);
  float* ssq = reinterpret_cast<float*>(ws + dp.ssq);
  int* gctx = reinterpret_cast<int*>(ws + pp.gctx);
  const int32_t* table_row = cache->block_table + (size_t)seq * cache->max_pages_per_seq;
  const long long pool_layer = (long long)cache->num_pages * m.nkv * 16 * m.d;

  for (int r0 = 0; r0 < n_tok; r0 += kPrefillChunkRows) {
    const int nv = std::min(kPrefillChunkRows, n_tok - r0);
    const int rows = cdiv(nv, 16) * 16, groups = rows / kQRows;
    // The plans of a shorter last chunk (same kernels, fewer m-blocks).
    const DraftPlan cp = rows == chunk_rows ? dp : prefill_layer_plan(m, groups, max_ctx);
    const int o_parts = residual_ssq_parts(cp.o, m.H / 16);
    const int dn_parts = residual_ssq_parts(cp.dn, m.H / 16);
    DF_TRY(launch_prefill_groups(cache->ctx_lens, seq, r0, groups, gctx, stream));
    {  // the fused features are the input rows: x = W_fuse . X
      const Plan fp = prefill_fuse_plan(m, nv);
      GemmParams g = base_params(fp, wb + P.w_fuse, 0, m.F / m.ktile,
                                 reinterpret_cast<const char*>(feats) + (size_t)r0 * m.F * m.es,
                                 m.F, nv, m.H / 16);
      g.a_kind = m.bf16 ? A_ROW_BF16 : A_ROW_F32;
      g.out = x;
      g.ldo = m.H;
      g.ksplit = fp.mt == kTallMT ? fp.ksub : 1;
      g.rows256 = fp.rows256;
      g.partial = reinterpret_cast<float*>(ws + pp.fpart);
      DF_TRY(launch_gemm(m.bf16, fp.mt, fp.npw, EPI_STORE, g, 1, stream));
    }
    DF_TRY(launch_prefill_rows(m.bf16, x, rows, nv, m.H,
                               reinterpret_cast<const float*>(wb + P.layer0 + P.attn_norm), xg,
                               ssq, stream));
    for (int l = 0; l < m.L; ++l) {
      const char* lb = wb + P.layer0 + (size_t)l * P.layer_stride;
      {  // RMSNorm + Q|K|V + RoPE; K/V of the valid rows into the cache (stored values)
        GemmParams g = base_params(cp.qkv, lb + P.wqkv, 0, m.H / m.ktile, xg, m.H, rows,
                                   (m.nq + 2 * m.nkv) * m.d / 16);
        g.a_kind = act_kind(m);
        g.norm = 1;
        g.ssq_in = ssq;
        g.ssq_parts = l == 0 ? 1 : dn_parts;
        g.ssq_ld = rows;
        g.eps = m.eps;
        g.q_out = reinterpret_cast<float*>(ws + cp.q);
        g.bk_out = reinterpret_cast<float*>(ws + cp.bk);
        g.bv_out = reinterpret_cast<float*>(ws + cp.bv);
        g.ctx_lens = gctx;
        g.rpr = kQRows;
        g.n_q = m.nq;
        g.n_kv = m.nkv;
        g.head_dim = m.d;
        set_rope(m, g);
        g.k_pool = reinterpret_cast<char*>(cache->k_pool) + (size_t)l * pool_layer * m.es;
        g.v_pool = reinterpret_cast<char*>(cache->v_pool) + (size_t)l * pool_layer * m.es;
        g.block_table = table_row;
        g.max_pages = cache->max_pages_per_seq;
        g.kv_rows = nv;
        g.ksplit = cp.qkv.mt == kTallMT ? cp.qkv.ksub : 1;
        g.partial = reinterpret_cast<float*>(ws + cp.kpart);
        DF_TRY(launch_gemm(m.bf16, cp.qkv.mt, cp.qkv.npw, EPI_QKV, g, 1, stream));
      }
      // The last layer's attention and MLP of the context rows feed nothing the draft reads.
      if (l + 1 == m.L) break;
      {  // causal attention: group g sees the cache up to its first row, then its own rows
        AttnArgs a{};
        a.q = reinterpret_cast<const float*>(ws + cp.q);
        a.bk = reinterpret_cast<const float*>(ws + cp.bk);
        a.bv = reinterpret_cast<const float*>(ws + cp.bv);
        a.k_pool = reinterpret_cast<const char*>(cache->k_pool) + (size_t)l * pool_layer * m.es;
        a.v_pool = reinterpret_cast<const char*>(cache->v_pool) + (size_t)l * pool_layer * m.es;
        a.block_table = table_row;
        a.table_ld = 0;
        a.max_pages = cache->max_pages_per_seq;
        a.ctx_lens = gctx;
        a.rpr = kQRows;
        a.nbk = kQRows;
        a.causal = 1;
        a.n_q = m.nq;
        a.n_kv = m.nkv;
        a.head_dim = m.d;
        a.nc = cp.nc;
        a.chunk = cp.chunk;
        a.scale = 1.0f / std::sqrt((float)m.d);
        a.part_o = reinterpret_cast<float*>(ws + cp.apart_o);
        a.part_ml = reinterpret_cast<float*>(ws + cp.apart_ml);
        a.out = ws + cp.ao;
        a.out_hilo = m.bf16;
        DF_TRY(launch_block_attention(m.bf16, a, groups, stream));
      }
      {  // output projection + residual
        GemmParams g = base_params(cp.o, lb + P.wo, 0, m.nq * m.d / m.ktile, ws + cp.ao,
                                   m.nq * m.d, rows, m.H / 16);
        g.a_kind = act_kind(m);
        g.out = x;
        g.ldo = m.H;
        g.xg_out = xg;
        g.gamma_next = reinterpret_cast<const float*>(lb + P.mlp_norm);
        g.ssq_out = ssq;
        g.ssq_ld = rows;
        g.ksplit = cp.o.mt == kTallMT ? cp.o.ksub : 1;
        g.partial = reinterpret_cast<float*>(ws + cp.kpart);
        DF_TRY(launch_gemm(m.bf16, cp.o.mt, cp.o.npw, EPI_RESIDUAL, g, 1, stream));
      }
      {  // RMSNorm + gate|up + SiLU * up
        GemmParams g = base_params(cp.gu, lb + P.wgu, 0, m.H / m.ktile, xg, m.H, rows,
                                   2 * m.I / 16);
        g.a_kind = act_kind(m);
        g.norm = 1;
        g.ssq_in = ssq;
        g.ssq_parts = o_parts;
        g.ssq_ld = rows;
        g.eps = m.eps;
        g.out = ws + cp.h;
        g.ldo = m.I;
        DF_TRY(launch_gemm(m.bf16, cp.gu.mt, cp.gu.npw, EPI_SWIGLU, g, 1, stream));
      }
      {  // down projection + residual; x * gain of the next layer's attention norm
        GemmParams g = base_params(cp.dn, lb + P.wd, 0, m.I / m.ktile, ws + cp.h, m.I, rows,
                                   m.H / 16);
        g.a_kind = act_kind(m);
        g.out = x;
        g.ldo = m.H;
        g.xg_out = xg;
        g.gamma_next = reinterpret_cast<const float*>(wb + P.layer0 +
                                                      (size_t)(l + 1) * P.layer_stride +
                                                      P.attn_norm);
        g.ssq_out = ssq;
        g.ssq_ld = rows;
        g.ksplit = cp.dn.mt == kTallMT ? cp.dn.ksub : 1;
        g.partial = reinterpret_cast<float*>(ws + cp.kpart);
        DF_TRY(launch_gemm(m.bf16, cp.dn.mt, cp.dn.npw, EPI_RESIDUAL, g, 1, stream));
      }
    }
  }
  return DFLASH_OK;
}

dflash_status dflash_draft_block(const dflash_config* cfg, const void* packed,
                                 const void* embed, const dflash_kv_cache* cache,
                                 const int32_t* anchor_ids, int32_t batch, int32_t* draft_ids,
                                 float* top2_gap, float* logits_out, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  Dims m;
  dflash_status st = check_config(cfg, &m);
  if (st != DFLASH_OK) return st;
  if ((st = check_cache(cache)) != DFLASH_OK) return st;
  if (!packed || !embed || !anchor_ids || !draft_ids || !workspace || batch <= 0)
    return DFLASH_ERR_INVALID_ARG;
  if ((long long)batch * m.rpr > kMaxBatch * 16 || cache->max_pages_per_seq > kMaxPagesPerSeq)
    return DFLASH_ERR_UNSUPPORTED;
  const int max_ctx = cache->max_pages_per_seq * 16;
  const DraftPlan dp = draft_plan(m, batch, max_ctx);
  if (ws_bytes < dp.total) return DFLASH_ERR_WORKSPACE;

  const Packed P = packed_layout(m);
  const char* wb = reinterpret_cast<const char*>(packed);
  char* ws = reinterpret_cast<char*>(workspace);
  float* x = reinterpret_cast<float*>(ws + dp.x);
  float* xg = reinterpret_cast<float*>(ws + dp.xg);
  float* ssq = reinterpret_cast<float*>(ws + dp.ssq);
  const int rows = batch * m.rpr;
  // Partial sums of squares per row left by the O projection (read by gate|up) and by the
  // down projection (read by the next Q|K|V and the LM head).
  const int o_parts = residual_ssq_parts(dp.o, m.H / 16);
  const int dn_parts = residual_ssq_parts(dp.dn, m.H / 16);
  const long long pool_layer = (long long)cache->num_pages * m.nkv * 16 * m.d;

  {  // x = embedding rows of [anchor, mask x 15]
    EmbedArgs e{};
    e.anchor_ids = anchor_ids;
    e.mask_id = m.mask;
    e.embed = embed;
    e.hidden = m.H;
    e.rpr = m.rpr;
    e.x = x;
    e.gamma = reinterpret_cast<const float*>(wb + P.layer0 + P.attn_norm);
    e.xg = xg;
    e.ssq = ssq;
    DF_TRY(launch_embed(m.bf16, e, rows, stream));
  }
  for (int l = 0; l < m.L; ++l) {
    const char* lb = wb + P.layer0 + (size_t)l * P.layer_stride;
    {  // RMSNorm + fused Q|K|V projection + RoPE
      GemmParams g = base_params(dp.qkv, lb + P.wqkv, 0, m.H / m.ktile, xg, m.H, rows,
                                 (m.nq + 2 * m.nkv) * m.d / 16);
      g.a_kind = act_kind(m);
      g.norm = 1;
      g.ssq_in = ssq;
      g.ssq_parts = l == 0 ? 1 : dn_parts;   // the embedding kernel leaves whole-row sums
      g.ssq_ld = rows;
      g.eps = m.eps;
      g.q_out = reinterpret_cast<float*>(ws + dp.q);
      g.bk_out = reinterpret_cast<float*>(ws + dp.bk);
      g.bv_out = reinterpret_cast<float*>(ws + dp.bv);
      g.ctx_lens = cache->ctx_lens;
      g.rpr = m.rpr;
      g.n_q = m.nq;
      g.n_kv = m.nkv;
      g.head_dim = m.d;
      set_rope(m, g);
      g.ksplit = dp.qkv.mt == kTallMT ? dp.qkv.ksub : 1;
      g.partial = reinterpret_cast<float*>(ws + dp.kpart);
      DF_TRY(launch_gemm(m.bf16, dp.qkv.mt, dp.qkv.npw, EPI_QKV, g, 1, stream));
    }
    {  // attention over injected context + block
      AttnArgs a{};
      a.q = reinterpret_cast<const float*>(ws + dp.q);
      a.bk = reinterpret_cast<const float*>(ws + dp.bk);
      a.bv = reinterpret_cast<const float*>(ws + dp.bv);
      a.k_pool = reinterpret_cast<const char*>(cache->k_pool) + (size_t)l * pool_layer * m.es;
      a.v_pool = reinterpret_cast<const char*>(cache->v_pool) + (size_t)l * pool_layer * m.es;
      a.block_table = cache->block_table;
      a.table_ld = cache->max_pages_per_seq;
      a.max_pages = cache->max_pages_per_seq;
      a.ctx_lens = cache->ctx_lens;
      a.rpr = m.rpr;
      a.nbk = m.nb;
      a.causal = 0;
      a.n_q = m.nq;
      a.n_kv = m.nkv;
      a.head_dim = m.d;
      a.nc = dp.nc;
      a.chunk = dp.chunk;
      a.scale = 1.0f / std::sqrt((float)m.d);
      a.part_o = reinterpret_cast<float*>(ws + dp.apart_o);
      a.part_ml = reinterpret_cast<float*>(ws + dp.apart_ml);
      a.out = ws + dp.ao;
      a.out_hilo = m.bf16;
      DF_TRY(launch_block_attention(m.bf16, a, rows / kQRows, stream));
    }
    {  // output projection + residual
      GemmParams g = base_params(dp.o, lb + P.wo, 0, m.nq * m.d / m.ktile, ws + dp.ao,
                                 m.nq * m.d, rows, m.H / 16);
      g.a_kind = act_kind(m);
      g.out = x;
      g.ldo = m.H;
      g.xg_out = xg;   // inputs of the MLP norm
      g.gamma_next = reinterpret_cast<const float*>(lb + P.mlp_norm);
      g.ssq_out = ssq;
      g.ssq_ld = rows;
      g.ksplit = dp.o.mt == kTallMT ? dp.o.ksub : 1;
      g.partial = reinterpret_cast<float*>(ws + dp.kpart);
      DF_TRY(launch_gemm(m.bf16, dp.o.mt, dp.o.npw, EPI_RESIDUAL, g, 1, stream));
    }
    {  // RMSNorm + gate|up + SiLU * up
      GemmParams g = base_params(dp.gu, lb + P.wgu, 0, m.H / m.ktile, xg, m.H, rows,
                                 2 * m.I / 16);
      g.a_kind = act_kind(m);
      g.norm = 1;
      g.ssq_in = ssq;
      g.ssq_parts = o_parts;
      g.ssq_ld = rows;
      g.eps = m.eps;
      g.out = ws + dp.h;
      g.ldo = m.I;
      DF_TRY(launch_gemm(m.bf16, dp.gu.mt, dp.gu.npw, EPI_SWIGLU, g, 1, stream));
    }
    {  // down projection + residual
      GemmParams g = base_params(dp.dn, lb + P.wd, 0, m.I / m.ktile, ws + dp.h, m.I, rows,
                                 m.H / 16);
      g.a_kind = act_kind(m);
      g.out = x;
      g.ldo = m.H;
      g.xg_out = xg;   // inputs of the next layer's attention norm, or of the final norm
      g.gamma_next = reinterpret_cast<const float*>(
          l + 1 < m.L ? wb + P.layer0 + (size_t)(l + 1) * P.layer_stride + P.attn_norm
                      : wb + P.final_norm);
      g.ssq_out = ssq;
      g.ssq_ld = rows;
      g.ksplit = dp.dn.mt == kTallMT ? dp.dn.ksub : 1;
      g.partial = reinterpret_cast<float*>(ws + dp.kpart);
      DF_TRY(launch_gemm(m.bf16, dp.dn.mt, dp.dn.npw, EPI_RESIDUAL, g, 1, stream));
    }
  }
  return launch_lm_head(m, P, wb, xg, ssq, dn_parts, rows, rows, true, draft_ids, top2_gap,
                        logits_out, reinterpret_cast<unsigned long long*>(ws + dp.keys), stream);
}

dflash_status dflash_lm_head_argmax(const dflash_config* cfg, const void* packed,
                                    const float* hidden, int32_t rows, int32_t* ids_out,
                                    float* logits_out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  Dims m;
  dflash_status st = check_config(cfg, &m);
  if (st != DFLASH_OK) return st;
  if (!packed || !hidden || !ids_out || !workspace || rows <= 0) return DFLASH_ERR_INVALID_ARG;
  if (rows > kMaxBatch * 16) return DFLASH_ERR_UNSUPPORTED;
  // The rows are first rewritten into the fragment layout, in the area a draft step keeps
  // its residual stream, so the LM head runs exactly the draft step's kernel.
  const size_t frag_bytes = align_up((size_t)cdiv(rows, 16) * 16 * m.H * 4);
  const size_t ssq_bytes = align_up((size_t)rows * 4);
  const size_t key_bytes = align_up(3 * lm_keys_bytes(m, rows));
  if (ws_bytes < kSyncBytes + frag_bytes + ssq_bytes + key_bytes) return DFLASH_ERR_WORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  float* xs = reinterpret_cast<float*>(ws + kSyncBytes);
  float* ssq = reinterpret_cast<float*>(ws + kSyncBytes + frag_bytes);
  auto* keys = reinterpret_cast<unsigned long long*>(ws + kSyncBytes + frag_bytes + ssq_bytes);
  const Packed P = packed_layout(m);
  const char* wb = reinterpret_cast<const char*>(packed);
  DF_TRY(launch_rows_to_fragments(hidden, rows, m.H, m.bf16,
                                  reinterpret_cast<const float*>(wb + P.final_norm), xs, ssq,
                                  stream));
  return launch_lm_head(m, P, wb, xs, ssq, 1, rows, rows, false, ids_out, nullptr, logits_out,
                        keys, stream);
}

static bool valid_block(int32_t block_size) {
  return block_size == 8 || block_size == 16 || block_size == 32;
}

dflash_status dflash_advance(const int32_t* accept_len, const int32_t* bonus, int32_t batch,
                             int32_t block_size, int32_t max_ctx, int32_t* ctx_lens,
                             int32_t* anchor_ids, int32_t* inject_seq, int32_t* inject_pos,
                             hipStream_t stream) {
  if (!accept_len || !bonus || !ctx_lens || !anchor_ids || !inject_seq || !inject_pos ||
      batch < 0 || !valid_block(block_size) || max_ctx < block_size)
    return DFLASH_ERR_INVALID_ARG;
  if (batch == 0) return DFLASH_OK;
  DF_TRY(launch_advance(accept_len, bonus, batch, block_size, max_ctx, ctx_lens, anchor_ids,
                        inject_seq, inject_pos, stream));
  return DFLASH_OK;
}

dflash_status dflash_verify_accept(const int32_t* draft_ids, const int32_t* target_ids,
                                   int32_t batch, int32_t block_size, int32_t* accept_len,
                                   int32_t* bonus, int32_t* emitted, hipStream_t stream) {
  if (!draft_ids || !target_ids || !accept_len || !bonus || batch < 0 ||
      !valid_block(block_size))
    return DFLASH_ERR_INVALID_ARG;
  if (batch == 0) return DFLASH_OK;
  DF_TRY(launch_verify_greedy(draft_ids, target_ids, batch, block_size, accept_len, bonus,
                              emitted, stream));
  return DFLASH_OK;
}

size_t dflash_verify_sampled_workspace_size(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0 || vocab > kMaxSampledVocab) return 0;
  return align_up(verify_sampled_stats_bytes(batch, vocab));
}

dflash_status dflash_verify_accept_sampled(const float* draft_logits,
                                           const float* target_logits, const float* u_draft,
                                           const float* u_accept, const float* u_resample,
                                           int32_t batch, int32_t vocab, int32_t* draft_ids,
                                           int32_t* accept_len, int32_t* emitted,
                                           void* workspace, size_t ws_bytes,
                                           hipStream_t stream) {
  if (!draft_logits || !target_logits || !u_draft || !u_accept || !u_resample || !draft_ids ||
      !accept_len || !emitted || !workspace || batch <= 0 || vocab <= 0)
    return DFLASH_ERR_INVALID_ARG;
  if (vocab > kMaxSampledVocab) return DFLASH_ERR_UNSUPPORTED;
  if (ws_bytes < dflash_verify_sampled_workspace_size(batch, vocab)) return DFLASH_ERR_WORKSPACE;
  SampledArgs a{};
  a.draft_logits = draft_logits;
  a.target_logits = target_logits;
  a.u_draft = u_draft;
  a.u_accept = u_accept;
  a.u_resample = u_resample;
  a.vocab = vocab;
  a.stats = reinterpret_cast<double*>(workspace);
  a.chunk_sums = a.stats + (size_t)batch * 31 * 2;
  a.chunks_ld = (vocab + 255) / 256;
  a.picks = reinterpret_cast<float*>(a.chunk_sums + (size_t)batch * a.chunks_ld);
  a.draft_ids = draft_ids;
  a.accept_len = accept_len;
  a.emitted = emitted;
  DF_TRY(launch_verify_sampled(a, batch, stream));
  return DFLASH_OK;
}

}  // extern "C"
