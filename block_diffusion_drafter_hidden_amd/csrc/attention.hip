// Block attention of the DFlash draft pass: the block queries of every head of one KV group
// attend, without a mask, to the request's injected context (paged KV cache) and to the
// block's own keys.
//
// Queries come in tiles of 16 rows (kQRows): a request has rpr = 16 rows (blocks of 8 or 16
// tokens; a block of 8 pads its request to 16 rows) or 32 rows (two tiles) and rpr block
// keys, of which the first nbk are valid.  The input-fusion prefill uses the same kernels
// with one tile per 16 context rows: each tile has the earlier rows as its cached context
// and its own 16 rows as block keys under a causal mask (row j sees block keys 0..j).
//
// Pass 1 (partials), grid (nc, n_kv, tiles): workgroup c covers context keys
// [c*chunk, min((c+1)*chunk, T_b)) (chunk a multiple of 32, at most kAttnMaxChunkKeys,
// fixed by the caller, so the page ids of a chunk are a few loads per lane issued before T_b
// arrives), and
// the last workgroup also the block keys (so a grid of nc * n_kv * tiles workgroups fills
// the chip in one round).  One wave per query head of the KV group.  Each wave keeps an
// online softmax (running max m, sum l, unnormalized output o) and writes (m, l, o).
// Pass 2 (merge), grid (n_q, d / 32, tiles): rescales the nc partials of each head to a
// common maximum and divides by the total sum, chunks in order, so results do not depend on
// scheduling.
//
// bf16 models run on 16x16x32 bf16 MFMA in transposed form, S^T = K Q^T and
// O^T += V^T P^T, so that every operand comes straight from memory or from the lane that
// computed it:
//   * a K fragment (16 keys x 32 dims) is one 16-byte load per lane from a K page
//     ([16 keys][d], row-major);
//   * a V^T fragment (16 dims x 32 keys) is two 8-byte loads per lane from the V pages,
//     which the cache keeps transposed ([d][16 keys]);
//   * the S^T output leaves lane l with keys 4*(l/16)+i of every 16-key page for query
//     row l%16 -- exactly the P^T fragment the PV product needs once the MFMA k index is
//     read as key (4*(l/16)+j) of the first page for j < 4 and of the second for j >= 4,
//     the same order the V^T fragment uses.
// GQA groups of at most 2 heads load these fragments straight from the pages (no LDS,
// no barriers); groups of 4 or more stage each 32-key step once per workgroup in
// double-buffered LDS (one barrier per step) and read the fragments from there.  Cache
// K/V are exact bf16 operands; fp32 queries, probabilities
// and block keys/values enter as hi + lo bf16 pairs (the lo x lo product, ~2^-32 relative,
// is dropped).  fp32 models use a VALU version of pass 1 with the same partial layout.
//
// Partial layout: part_o[slot][head_in_group][dt][q][row][i] holds output dim
// 16*dt + 4*q + i of block row `row` (a float4 per (dt, q, row)); part_ml[slot][head][row]
// holds (m, l).  slot = (tile * n_kv + g) * nc + c.
#include <type_traits>

#include "attention.h"
#include "common.h"

namespace dflash {


__device__ inline long long part_o_index(long long slot, int G, int hh, int D, int row,
                                         int dim) {
  return ((((slot * G + hh) * (D / 16) + dim / 16) * 4 + (dim % 16) / 4) * kQRows + row) * 4 +
         dim % 4;
}

// 8 floats -> hi and lo bf16 fragments (pairs rounded by one packed convert each).
__device__ inline void split8(const float (&f)[8], i32x4& hi, i32x4& lo) {
  int h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = f[2 * i], b = f[2 * i + 1];
    h[i] = bf16_pair_split(a, b);
    l[i] = bf16_pair(a, b);
  }
  hi = i32x4{h[0], h[1], h[2], h[3]};
  lo = i32x4{l[0], l[1], l[2], l[3]};
}

// Zero the bf16 keys of a V^T fragment that lie at or beyond `nk` valid keys of the
// 32-key step (element j is key 4q + j of the first page for j < 4, 16 + 4q + j - 4 else).
__device__ inline i32x4 mask_vt(i32x4 v, int q, int nk) {
  bf16x8 e = __builtin_bit_cast(bf16x8, v);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = (j < 4 ? 0 : 16) + 4 * q + (j & 3);
    if (key >= nk) e[j] = (bf16)0.f;
  }
  return __builtin_bit_cast(i32x4, e);
}

typedef __attribute__((address_space(1))) void* global_void_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Scores are kept in base-2 units: the queries are scaled by log2(e) / sqrt(d), so every
// exponential is a plain exp2 and partial maxima m are log2-scaled (the merge uses exp2 too).
constexpr float kLog2e = 1.4426950408889634f;
// The running reference maximum m of a row is raised only when a score exceeds it by more
// than this (in base-2 units), so probabilities exp2(s - m) stay below 2^8 and the
// accumulator is rescaled rarely; (m, l, o) remain an exact representation of the softmax
// state for any reference.
constexpr float kRescaleSlack = 8.0f;

// Maximum / sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48):
// each row-swap permute hands every lane its partner row's value, so after the 16- and the
// 32-lane swap every lane holds the same result (both operands of each step commute).
__device__ inline float rows_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ inline float rows_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA partials.  One wave per query head of the group; the per-head state and the
// math of one 32-key step are shared by two kernels that differ in how K/V reach the wave:
//   attn_partial_bf16  (G <= 2): every wave loads its step fragments straight from the
//                      paged cache into registers;
//   attn_partial_lds   (G >= 4): the workgroup loads each step once, as coalesced 16-byte
//                      pieces spread over all its threads, into an LDS double buffer that
//                      the G head waves then read (G times less cache traffic).
// ------------------------------------------------------------------------------------------
template <int D>
struct HeadState {
  static constexpr int KS = D / 32;   // dim steps of S^T
  static constexpr int DT = D / 16;   // dim tiles of O^T
  i32x4 qf[KS][2];                    // Q^T fragments (hi, lo), base-2 scaled
  f32x4 o[DT];                        // O^T accumulator: dims 16dt + 4q + i of block row n
  float m_run;                        // the row's reference maximum (same in its 4 lanes)
  float l_run;                        // this lane's part of the row's sum (its keys only)
  int q;                              // lane / 16

  __device__ void init(const f32x4 (&qraw)[KS][2], float qscale, int lane) {
    q = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 v0 = qraw[ks][0] * qscale, v1 = qraw[ks][1] * qscale;
      const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      split8(f, qf[ks][0], qf[ks][1]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // Online-softmax update for one 32-key step given S^T tiles s[2] (lane: keys
  // 16 pg + 4q + i for query n); returns the P^T fragment (hi, lo).  The accumulator is
  // rescaled only when some row's maximum passed its reference by kRescaleSlack (a branch
  // uniform over the wave).  Only a kMasked step (the last of a chunk, or the block) can
  // hold fewer than 32 valid keys.
  template <bool kMasked>
  __device__ void softmax(const f32x4 (&s)[2], int nk, i32x4& p_hi, i32x4& p_lo) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e / 4][e % 4];
    if (kMasked) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (16 * (e / 4) + 4 * q + e % 4 >= nk) x[e] = -INFINITY;
    }
    const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    // The row maximum is formed only when some lane's scores pass its reference by the
    // slack (a branch uniform over the wave; always on the first step).
    if (__ballot(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, rows_max(mx));   // finite: key 0 of a step is valid
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first step
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
    if (kMasked) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (16 * (e / 4) + 4 * q + e % 4 >= nk) pv[e] = 0.f;
    }
    // The lane keeps its own part of the row sum; the four lanes of a row are added once,
    // when the partial is stored.
    l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    split8(pv, p_hi, p_lo);
  }

  // One 32-key step: k[pg][ks] is the K fragment (16 keys of page pg x dims 32ks + 8q..+8),
  // v[dt] the V^T fragment of dim 16dt + n: keys 4q..4q+3 of page 0, then of page 1.
  template <bool kMasked>
  __device__ void step(const i32x4 (&k)[2][KS], const i32x4 (&v)[DT], int nk) {
    // d = 128: Q hi and Q lo products accumulate separately (four independent MFMA chains
    // of four); d = 64: one chain per page (two chains of four, no adds).
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (KS > 2) {
      f32x4 sl[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          s[pg] = mfma_tile<bf16>(k[pg][ks], qf[ks][0], s[pg]);
          sl[pg] = mfma_tile<bf16>(k[pg][ks], qf[ks][1], sl[pg]);
        }
      s[0] += sl[0];
      s[1] += sl[1];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          s[pg] = mfma_tile<bf16>(k[pg][ks], qf[ks][0], s[pg]);
          s[pg] = mfma_tile<bf16>(k[pg][ks], qf[ks][1], s[pg]);
        }
    }
    i32x4 ph, pl;
    softmax<kMasked>(s, nk, ph, pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      i32x4 vv = v[dt];
      if (kMasked) vv = mask_vt(vv, q, nk);   // stale cache slots may hold any bits
      o[dt] = mfma_tile<bf16>(vv, ph, o[dt]);
      o[dt] = mfma_tile<bf16>(vv, pl, o[dt]);
    }
  }

  // The RPR block keys from LDS (fp32 K [RPR][D], then V^T [D][RPR]; RPR = 16 or 32, the
  // second 16 on the S^T tile of page 1), hi + lo on both operands.  Lane n (query row n of
  // the tile) takes block keys below nk, its own limit (the valid keys, or the causal bound).
  template <int RPR>
  __device__ void block(const char* blk_s, int n, int nk) {
    const float* bk_s = reinterpret_cast<const float*>(blk_s);
    const float* bv_s = reinterpret_cast<const float*>(blk_s + RPR * D * 4);
    constexpr int NP = RPR / 16;   // 16-key pages of the block
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int pg = 0; pg < NP; ++pg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float* kr = bk_s + (16 * pg + n) * D + ks * 32 + q * 8;
        const f32x4 k0 = *reinterpret_cast<const f32x4*>(kr);
        const f32x4 k1 = *reinterpret_cast<const f32x4*>(kr + 4);
        const float f[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        i32x4 kh, kl;
        split8(f, kh, kl);
        s[pg] = mfma_tile<bf16>(kh, qf[ks][0], s[pg]);
        s[pg] = mfma_tile<bf16>(kh, qf[ks][1], s[pg]);
        s[pg] = mfma_tile<bf16>(kl, qf[ks][0], s[pg]);
      }
    i32x4 ph, pl;
    softmax<true>(s, nk, ph, pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float* vr = bv_s + (16 * dt + n) * RPR + q * 4;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(vr);
      f32x4 v1 = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NP == 2) v1 = *reinterpret_cast<const f32x4*>(vr + 16);
      const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      i32x4 vh, vl;
      split8(f, vh, vl);
      o[dt] = mfma_tile<bf16>(vh, ph, o[dt]);
      o[dt] = mfma_tile<bf16>(vh, pl, o[dt]);
      o[dt] = mfma_tile<bf16>(vl, ph, o[dt]);
    }
  }

  // Partial of this chunk (layout in the file header).
  __device__ void store(const AttnArgs& a, long long slot, int G, int hh, int n) const {
    f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + (slot * G + hh) * (DT * 4 * kQRows);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) po[(dt * 4 + q) * kQRows + n] = o[dt];
    const float l_row = rows_sum(l_run);
    if (q == 0) {
      float* ml = a.part_ml + ((slot * G + hh) * kQRows + n) * 2;
      ml[0] = m_run;
      ml[1] = l_row;
    }
  }
};

// Everything a partial workgroup needs before its first step: the chunk's key range, the
// page ids (lane i: logical page i of the chunk, at most 64, clamped into the table row and
// fetched together with T_b), the block K/V copied into LDS by the last chunk's workgroup,
// this wave's Q rows, and the lane's limit on the block keys.
template <int D>
struct ChunkSetup {
  int kbeg, kend, npg, nsteps;
  int pid[kAttnPidRegs];   // pid[r] in lane i: physical page of logical page 64 r + i
  bool has_block;
  int blk_nk;              // block keys below this index are seen by the lane's query row
};

// Request of tile `tile` (rpr / 16 tiles per request) and the lane's block-key limit for
// query row n of the tile.
__device__ inline int tile_request(const AttnArgs& a, int tile) { return tile * kQRows / a.rpr; }
__device__ inline int block_key_limit(const AttnArgs& a, int tile, int n) {
  const int row = tile * kQRows % a.rpr + n;   // row of the request's block
  return a.causal ? min(a.nbk, row + 1) : a.nbk;
}

template <int D, int G, int RPR>
__device__ inline ChunkSetup<D> chunk_setup(const AttnArgs& a, char* blk_s,
                                            f32x4 (&qraw)[D / 32][2]) {
  constexpr int kBlockBytes = RPR * D * 4;           // the block's K, or its V^T, in fp32
  constexpr int kCopies = 2 * kBlockBytes / 1024;    // 1 KB (64 lanes x 16 B) per copy
  static_assert(kCopies % G == 0, "block copies split evenly over the waves");
  const int c = blockIdx.x, g = blockIdx.y, tile = blockIdx.z;
  const int b = tile_request(a, tile);
  const int lane = threadIdx.x % kWave, hh = threadIdx.x / kWave;
  const int n = lane & 15, q = lane >> 4;
  ChunkSetup<D> cs;
  cs.blk_nk = block_key_limit(a, tile, n);
  const int kbeg0 = c * a.chunk;
  const int* table = a.block_table + (long long)b * a.table_ld;
  int pid[kAttnPidRegs];
#pragma unroll
  for (int r = 0; r < kAttnPidRegs; ++r)
    pid[r] = table[min(kbeg0 / kPage + r * kWave + lane, a.max_pages - 1)];
  const int T_b = a.ctx_lens[b];
  cs.has_block = c == a.nc - 1;
  cs.kbeg = min(kbeg0, T_b);
  cs.kend = min(kbeg0 + a.chunk, T_b);

  // The last chunk's workgroup copies the block's fp32 keys [RPR][d] and transposed values
  // [d][RPR] (contiguous per KV group) into LDS with direct loads, which need no registers.
  // The other workgroups issue the same copies from the first kilobyte of the arrays (and
  // never read them), so that every wave's load count is the same on every path.
  {
    const long long grp = cs.has_block ? (long long)(b * a.n_kv + g) * kBlockBytes : 0;
    const char* srck = reinterpret_cast<const char*>(a.bk) + grp;
    const char* srcv = reinterpret_cast<const char*>(a.bv) + grp;
#pragma unroll
    for (int j = 0; j < kCopies / G; ++j) {
      const int i = hh + j * G;
      const int half = i / (kCopies / 2), off = (i % (kCopies / 2)) * 1024;
      const char* src = (half ? srcv : srck) + (cs.has_block ? off : 0) + lane * 16;
      __builtin_amdgcn_global_load_lds((global_void_ptr)src,
                                       (lds_void_ptr)(blk_s + half * kBlockBytes + off), 16, 0,
                                       0);
    }
  }
  // Issue all of the above before the page ids are waited for (the compiler waits for every
  // outstanding load once a direct-to-LDS load is pending, so that first wait retires them).
  __builtin_amdgcn_sched_barrier(0);

  // Q^T rows of this head (B operand of S^T): lane holds block row n, dims 32*ks + 8q .. +8.
  const float* src = a.q + ((long long)(tile * kQRows + n) * a.n_q + g * G + hh) * D + q * 8;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qraw[ks][0] = *reinterpret_cast<const f32x4*>(src + ks * 32);
    qraw[ks][1] = *reinterpret_cast<const f32x4*>(src + ks * 32 + 4);
  }
  cs.npg = (cs.kend - cs.kbeg + kPage - 1) / kPage;   // 0 .. kAttnMaxChunkKeys / 16
  cs.nsteps = (cs.kend - cs.kbeg + 31) / 32;
  // A page past the chunk's last is read from the last one (its keys are masked), and an
  // empty chunk reads physical page 0 and uses nothing.
#pragma unroll
  for (int r = 0; r < kAttnPidRegs; ++r) cs.pid[r] = cs.npg > 0 ? pid[r] : 0;
  return cs;
}

// Physical page of the chunk's logical page li (wave-uniform li), clamped as above.  The
// index arithmetic is made scalar (li is uniform), so a lookup is a readlane per page-id
// register and scalar selects.
template <int D>
__device__ inline long long chunk_page(const ChunkSetup<D>& cs, int li) {
  li = __builtin_amdgcn_readfirstlane(li);
  const int npg = __builtin_amdgcn_readfirstlane(cs.npg);
  const int lc = max(min(li, npg - 1), 0), reg = lc / kWave, ln = lc % kWave;
  int page = __builtin_amdgcn_readlane(cs.pid[0], ln);
#pragma unroll
  for (int r = 1; r < kAttnPidRegs; ++r) {
    const int v = __builtin_amdgcn_readlane(cs.pid[r], ln);
    page = reg == r ? v : page;
  }
  return page;
}

template <int D>
struct StepRegs {
  i32x4 k[2][D / 32];      // two pages x dim steps
  i32x2 v[D / 16][2];      // dim tiles x pages
  int nk;                  // valid keys of the step (1..32)
};

template <int D, int G, int RPR>
__global__ __launch_bounds__(G * kWave, 2) void attn_partial_bf16(AttnArgs a) {
  constexpr int KS = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(16))) char blk_s[2 * RPR * D * 4];   // K, then V^T
  const int g = blockIdx.y;
  const int lane = threadIdx.x % kWave, hh = threadIdx.x / kWave;
  const int n = lane & 15, q = lane >> 4;
  const int nkv = a.n_kv;
  f32x4 qraw[KS][2];
  const ChunkSetup<D> cs = chunk_setup<D, G, RPR>(a, blk_s, qraw);

  const bf16* kpool = reinterpret_cast<const bf16*>(a.k_pool);
  const bf16* vpool = reinterpret_cast<const bf16*>(a.v_pool);
  // Step st reads logical pages 2st and 2st+1 of the chunk.  Every step issues the same
  // loads with no branch, so the compiler can wait for one step's loads while the next
  // step's stay in flight.
  auto load_step = [&](int st, StepRegs<D>& r) {
    r.nk = min(32, cs.kend - cs.kbeg - 32 * st);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const long long page = chunk_page(cs, 2 * st + pg);
      const bf16* kp = kpool + ((page * nkv + g) * kPage + n) * D + q * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) r.k[pg][ks] = *reinterpret_cast<const i32x4*>(kp + ks * 32);
      const bf16* vp = vpool + ((page * nkv + g) * D + n) * kPage + q * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        r.v[dt][pg] = *reinterpret_cast<const i32x2*>(vp + dt * 16 * kPage);
    }
  };
  // Two register sets: while one step's math runs, the next step's loads are in flight.
  StepRegs<D> ra, rb;
  load_step(0, ra);
  load_step(min(1, max(cs.nsteps - 1, 0)), rb);
  __builtin_amdgcn_sched_barrier(0);   // keep every prologue load ahead of the math below

  HeadState<D> hs;
  hs.init(qraw, a.scale * kLog2e, lane);
  const int nsteps = cs.nsteps;
  // Steady state: ra holds step st, rb step st + 1, and both prefetches exist.
  int st = 0;
  // Steps of the steady state are full (at least two more follow them); the tail takes the
  // masked form, since its last step may be the chunk's partial one.
  auto vfrags = [](const StepRegs<D>& r, i32x4 (&v)[DT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      v[dt] = i32x4{r.v[dt][0][0], r.v[dt][0][1], r.v[dt][1][0], r.v[dt][1][1]};
  };
  auto full_step = [&](const StepRegs<D>& r) {
    i32x4 v[DT];
    vfrags(r, v);
    hs.template step<false>(r.k, v, r.nk);
  };
  auto tail_step = [&](const StepRegs<D>& r) {
    i32x4 v[DT];
    vfrags(r, v);
    hs.template step<true>(r.k, v, r.nk);
  };
  for (; st + 3 < nsteps; st += 2) {
    full_step(ra);
    load_step(st + 2, ra);
    full_step(rb);
    load_step(st + 3, rb);
  }
  // 0..3 steps remain.
  if (st < nsteps) tail_step(ra);
  if (st + 2 < nsteps) load_step(st + 2, ra);
  if (st + 1 < nsteps) tail_step(rb);
  if (st + 2 < nsteps) tail_step(ra);

  if (cs.has_block) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    hs.template block<RPR>(blk_s, n, cs.blk_nk);
  }
  hs.store(a, ((long long)blockIdx.z * nkv + g) * a.nc + blockIdx.x, G, hh, n);
}

// ------------------------------------------------------------------------------------------
// LDS-staged variant (G >= 4).  A step (two pages of K and of V, 128 d bytes) is loaded as
// 16-byte pieces, d / (8 G) per thread: piece p of the step (p = j * 64G + thread) is bytes
// 16 (p mod 2d) .. +16 of quarter p / 2d, the quarters being K page 0, K page 1, V page 0
// and V page 1 (32 d bytes each, contiguous in the cache).  Pieces are staged in registers
// RS steps ahead and written to an LDS double buffer, XOR-swizzled so that the fragment
// reads hit distinct banks:
//   K row r (2d bytes): 16-byte piece j sits at piece j ^ swz(r), swz(r) = r & 15 (d = 128)
//                       or (r >> 1) & 7 (d = 64);
//   V rows of both pages interleaved: row `dim` is 64 bytes, 16-byte chunk c holding keys
//   4c'..4c'+3 of page 0 then of page 1 for c' = c ^ ((dim >> 2) & 3) -- exactly one V^T
//   MFMA fragment, so a lane's fragment is one 16-byte read.
// One barrier per step: after it, the stage holding step t is complete and every wave has
// finished reading step t - 1, whose stage the step-(t + 1) pieces then overwrite.
// ------------------------------------------------------------------------------------------
template <int D, int G>
struct LdsStep {
  static constexpr int kStepBytes = 128 * D;              // K + V of 32 keys
  static constexpr int kQuarter = 32 * D;                 // one page of K or of V
  static constexpr int kPieces = kStepBytes / 16;
  static constexpr int kThreads = G * kWave;
  static constexpr int NL = kPieces / kThreads;           // 16-byte loads per thread
  static_assert(kPieces % kThreads == 0, "pieces split evenly over the threads");
  static_assert((2 * D) % kWave == 0, "a wave's 64 pieces stay inside one quarter");
};

template <int D>
__device__ inline int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

template <int D, int G, int RPR>
__global__ __launch_bounds__(G * kWave, (D == 64 && G == 8) ? 4 : 2) void attn_partial_lds(
    AttnArgs a) {
  using L = LdsStep<D, G>;
  constexpr int KS = D / 32, DT = D / 16, NL = L::NL;
  // Register stages (steps ahead).  d = 64 with G = 8 runs two workgroups per CU (four
  // waves per SIMD, at most 128 registers), which needs the shallower ring (three stages fit
  // but measured slower: gpt-oss batch 128 20.79 -> 21.64 ms per step).
  constexpr int RS = (D == 64 && G == 8) ? 2 : 4;
  __shared__ __attribute__((aligned(16))) char blk_s[2 * RPR * D * 4];
  __shared__ __attribute__((aligned(16))) char kv_s[2][L::kStepBytes];
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave, hh = tid / kWave;
  const int n = lane & 15, q = lane >> 4;
  const int nkv = a.n_kv;
  f32x4 qraw[KS][2];
  const ChunkSetup<D> cs = chunk_setup<D, G, RPR>(a, blk_s, qraw);
  const int nsteps = cs.nsteps;

  // Static description of this thread's pieces: quarter (page, K or V), source byte offset
  // inside the page's K or V block, and LDS byte offsets inside a stage (V pieces: the two
  // 8-byte halves go to two places).
  int src_off[NL], dst_off[NL], dst_off2[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int p = j * L::kThreads + tid;
    const int quarter = p / (2 * D), e = p % (2 * D);
    int dst;
    if (quarter < 2) {                  // K: row r, piece jj
      const int r = e / (D / 8), jj = e % (D / 8);
      src_off[j] = e * 16;
      dst = r * 2 * D + ((jj ^ k_swz<D>(r)) * 16);
    } else {                            // V^T: row dim, keys 8h .. 8h+7 of page quarter - 2
      const int dim = e / 2, h = e % 2, pg = quarter - 2, sw = (dim >> 2) & 3;
      src_off[j] = e * 16;
      dst = 2 * L::kQuarter + dim * 64 + (((2 * h) ^ sw) * 16) + pg * 8;
      dst_off2[j] = 2 * L::kQuarter + dim * 64 + (((2 * h + 1) ^ sw) * 16) + pg * 8;
    }
    dst_off[j] = quarter < 2 ? quarter * L::kQuarter + dst : dst;
  }
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  auto load_pieces = [&](int st, i32x4 (&r)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      // quarter is uniform over the wave (a wave's 64 pieces lie inside one quarter)
      const int quarter = (j * L::kThreads + hh * kWave) / (2 * D);
      const long long page = chunk_page(cs, 2 * st + (quarter & 1));
      const char* base = (quarter < 2 ? kbase : vbase) + (page * nkv + g) * (long long)L::kQuarter;
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + src_off[j]));
    }
  };
  auto store_pieces = [&](int stage, const i32x4 (&r)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if ((j * L::kThreads + hh * kWave) / (2 * D) < 2) {   // K (uniform over the wave)
        *reinterpret_cast<i32x4*>(kv_s[stage] + dst_off[j]) = r[j];
      } else {
        *reinterpret_cast<i32x2*>(kv_s[stage] + dst_off[j]) = i32x2{r[j][0], r[j][1]};
        *reinterpret_cast<i32x2*>(kv_s[stage] + dst_off2[j]) = i32x2{r[j][2], r[j][3]};
      }
    }
  };
  // Fragments of one step from a stage: K as in attn_partial_bf16; a V^T fragment (both
  // pages' keys 4q..4q+3 of one dim) is one 16-byte read.
  auto compute = [&](HeadState<D>& hs, int stage, int st, auto masked) {
    const char* sb = kv_s[stage];
    i32x4 k[2][KS], v[DT];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        k[pg][ks] = *reinterpret_cast<const i32x4*>(
            sb + pg * L::kQuarter + n * 2 * D + (((ks * 4 + q) ^ k_swz<D>(n)) * 16));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dim = 16 * dt + n;
      v[dt] = *reinterpret_cast<const i32x4*>(sb + 2 * L::kQuarter + dim * 64 +
                                              ((q ^ ((dim >> 2) & 3)) * 16));
    }
    hs.template step<decltype(masked)::value>(k, v, min(32, cs.kend - cs.kbeg - 32 * st));
  };

  i32x4 rs[RS][NL];
  // Prologue: steps 0 .. RS-1 in flight (with no branch: a step past the last repeats it),
  // step 0 staged.
#pragma unroll
  for (int s = 0; s < RS; ++s) load_pieces(min(s, max(nsteps - 1, 0)), rs[s]);
  __builtin_amdgcn_sched_barrier(0);
  HeadState<D> hs;
  hs.init(qraw, a.scale * kLog2e, lane);
  if (nsteps > 0) store_pieces(0, rs[0]);
  __syncthreads();

  // Steady state, RS steps per trip: every load issued here is of a real step.
  int t = 0;
  for (; t + 2 * RS <= nsteps; t += RS) {
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      load_pieces(t + i + RS, rs[i]);
      compute(hs, (t + i) & 1, t + i, std::false_type{});   // RS more steps follow: full
      store_pieces((t + i + 1) & 1, rs[(i + 1) % RS]);
      __syncthreads();
    }
  }
  // Tail: fewer than 2 RS steps remain; step t + i is in register set i % RS.  Every step
  // but the chunk's last is full; the last (possibly partial) one is taken after the loop
  // from its LDS stage.
#pragma unroll
  for (int i = 0; i < 2 * RS - 1; ++i) {
    if (t + i + 1 < nsteps) {
      if (i < RS && t + i + RS < nsteps) load_pieces(t + i + RS, rs[i % RS]);
      compute(hs, (t + i) & 1, t + i, std::false_type{});
      store_pieces((t + i + 1) & 1, rs[(i + 1) % RS]);
      __syncthreads();
    }
  }
  if (nsteps > 0) compute(hs, (nsteps - 1) & 1, nsteps - 1, std::true_type{});

  if (cs.has_block) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    hs.template block<RPR>(blk_s, n, cs.blk_nk);
  }
  hs.store(a, ((long long)blockIdx.z * nkv + g) * a.nc + blockIdx.x, G, hh, n);
}

// ------------------------------------------------------------------------------------------
// fp32: VALU partial kernel (rows r = head*16 + slot)
// ------------------------------------------------------------------------------------------
constexpr int kKeys = 32;       // keys per step
constexpr int kThreads = 256;   // 4 waves

template <int D, int R>
__global__ __launch_bounds__(kThreads) void attn_partial_f32(AttnArgs a) {
  constexpr int G = R / kQRows;
  constexpr int OPH = kThreads / D;
  constexpr int NRO = R / OPH;
  constexpr int SPH = kThreads / kKeys;
  constexpr int NRS = R / SPH;
  __shared__ float q_s[R][D + 1];
  __shared__ float k_s[kKeys][D + 1];
  __shared__ float v_s[kKeys][D];
  __shared__ float p_s[R][kKeys + 1];
  __shared__ float m_s[R], l_s[R], sc_s[R];

  const int c = blockIdx.x, g = blockIdx.y, tile = blockIdx.z;
  const int b = tile_request(a, tile);
  const int tid = threadIdx.x;
  const int nq = a.n_q, nkv = a.n_kv, rpr = a.rpr;
  const int T_b = a.ctx_lens[b];
  const bool has_block = c == a.nc - 1;
  const float qscale = a.scale * kLog2e;   // base-2 scores, as in the MFMA kernel
  const int kbeg = min(c * a.chunk, T_b);
  const int kend = min(kbeg + a.chunk, T_b);
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, i = idx % D;
    const int hh = r / kQRows, j = r % kQRows;
    q_s[r][i] = a.q[((long long)(tile * kQRows + j) * nq + g * G + hh) * D + i] * qscale;
  }
  if (tid < R) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float o[NRO];
#pragma unroll
  for (int n = 0; n < NRO; ++n) o[n] = 0.f;
  __syncthreads();

  const float* kpool = reinterpret_cast<const float*>(a.k_pool);
  const float* vpool = reinterpret_cast<const float*>(a.v_pool);
  // Context steps of 32 keys, then (last workgroup) one step over the rpr block keys (at
  // most 32), of which row r sees those below block_key_limit.
  const int n_ctx_steps = (kend - kbeg + kKeys - 1) / kKeys;
  for (int st = 0; st < n_ctx_steps + (has_block ? 1 : 0); ++st) {
    const bool is_block = st == n_ctx_steps;
    const int k0 = is_block ? 0 : kbeg + st * kKeys;
    const int nk = is_block ? rpr : min(kKeys, kend - k0);
    for (int idx = tid; idx < kKeys * D; idx += kThreads) {
      const int kk = idx / D, i = idx % D;
      float kv = 0.f, vv = 0.f;
      if (kk < nk) {
        const int t = k0 + kk;
        if (is_block) {
          kv = a.bk[((long long)(b * nkv + g) * rpr + t) * D + i];
          vv = a.bv[((long long)(b * nkv + g) * D + i) * rpr + t];
        } else {
          const long long page = a.block_table[(long long)b * a.table_ld + t / kPage];
          kv = kpool[((page * nkv + g) * kPage + t % kPage) * D + i];
          vv = vpool[((page * nkv + g) * D + i) * kPage + t % kPage];
        }
      }
      k_s[kk][i] = kv;
      v_s[kk][i] = vv;
    }
    __syncthreads();
    {
      const int cc = tid % kKeys, r0 = tid / kKeys;
      float s[NRS];
#pragma unroll
      for (int n = 0; n < NRS; ++n) s[n] = 0.f;
      for (int i = 0; i < D; ++i) {
        const float kv = k_s[cc][i];
#pragma unroll
        for (int n = 0; n < NRS; ++n) s[n] += q_s[r0 + n * SPH][i] * kv;
      }
#pragma unroll
      for (int n = 0; n < NRS; ++n) {
        const int r = r0 + n * SPH;
        const int lim = is_block ? block_key_limit(a, tile, r % kQRows) : nk;
        p_s[r][cc] = cc < lim ? s[n] : -INFINITY;
      }
    }
    __syncthreads();
    if (tid < R) {
      const float mold = m_s[tid];
      float mx = mold;
      for (int cc = 0; cc < nk; ++cc) mx = fmaxf(mx, p_s[tid][cc]);
      const float sc = exp2f(mold - mx);
      float l = l_s[tid] * sc;
      for (int cc = 0; cc < kKeys; ++cc) {
        const float pe = cc < nk ? exp2f(p_s[tid][cc] - mx) : 0.f;
        p_s[tid][cc] = pe;
        l += pe;
      }
      m_s[tid] = mx;
      l_s[tid] = l;
      sc_s[tid] = sc;
    }
    __syncthreads();
    {
      const int i = tid % D, r0 = tid / D;
#pragma unroll
      for (int n = 0; n < NRO; ++n) {
        const int r = r0 + n * OPH;
        float acc = o[n] * sc_s[r];
        for (int cc = 0; cc < kKeys; ++cc) acc += p_s[r][cc] * v_s[cc][i];
        o[n] = acc;
      }
    }
    __syncthreads();
  }
  const long long slot = ((long long)tile * nkv + g) * a.nc + c;
  const int i = tid % D, r0 = tid / D;
#pragma unroll
  for (int n = 0; n < NRO; ++n) {
    const int r = r0 + n * OPH;
    a.part_o[part_o_index(slot, G, r / kQRows, D, r % kQRows, i)] = o[n];
  }
  if (tid < R) {
    a.part_ml[(slot * R + tid) * 2 + 0] = m_s[tid];
    a.part_ml[(slot * R + tid) * 2 + 1] = l_s[tid];
  }
}

// ------------------------------------------------------------------------------------------
// Merge: one workgroup per (query head, 32-dim slice, request), one thread per float4 of the
// slice (16 rows x 32 dims).  The slice's partials of the first kMergeBatch chunks are loaded
// before the (m, l) pass so both travel in one round trip; the per-row maximum and sum come
// from 16 rows x 8 chunk lanes through LDS; the weighted sum runs over chunks in order.  The
// result is written in the layout the output projection reads.
// ------------------------------------------------------------------------------------------
constexpr int kMergeThreads = 128;   // float4s of a 16 x 32 slice

// NCMAX: the most chunks the instance takes (its LDS weights and its loads in flight are
// sized by it; 16 covers every plan but very long contexts at small batch).
template <int D, int NCMAX>
__global__ __launch_bounds__(kMergeThreads) void attn_merge(AttnArgs a) {
  constexpr int kMergeBatch = NCMAX < 40 ? NCMAX : 40;
  constexpr int NCL = kMergeThreads / kQRows;   // chunk lanes per row
  constexpr int NT = D * 4;                     // float4s of one head's 16 x D partial
  __shared__ float w_s[NCMAX + 1][kQRows];
  __shared__ float m_s[NCMAX + 1][kQRows];
  __shared__ float red[NCL][kQRows];
  __shared__ float M_s[kQRows], invL_s[kQRows];
  const int h = blockIdx.x, slice = blockIdx.y, tile = blockIdx.z;
  const int G = a.n_q / a.n_kv;
  const int g = h / G, hh = h % G;
  const int nch = a.nc;
  const long long slot0 = ((long long)tile * a.n_kv + g) * nch;
  const int tid = threadIdx.x;
  const int f = slice * kMergeThreads + tid;     // float4 index (dt, q, row) within the head
  const long long cstride = (long long)G * NT;   // float4s between chunks
  const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o) + (slot0 * G + hh) * NT + f;

  f32x4 v[kMergeBatch];
#pragma unroll
  for (int c = 0; c < kMergeBatch; ++c)
    v[c] = c < nch ? src[c * cstride] : f32x4{0.f, 0.f, 0.f, 0.f};

  // Row maximum and weights.  Thread (row j, chunk lane cl).
  const int j = tid % kQRows, cl = tid / kQRows;
  float mx = -INFINITY;
  for (int c = cl; c < nch; c += NCL) {
    const float* ml = a.part_ml + (((slot0 + c) * G + hh) * kQRows + j) * 2;
    const float m = ml[0], l = ml[1];
    const float mm = l > 0.f ? m : -INFINITY;   // empty chunks carry no weight
    m_s[c][j] = mm;
    w_s[c][j] = l;
    mx = fmaxf(mx, mm);
  }
  red[cl][j] = mx;
  __syncthreads();
  if (tid < kQRows) {
    float M = -INFINITY;
    for (int r = 0; r < NCL; ++r) M = fmaxf(M, red[r][tid]);
    M_s[tid] = M;
  }
  __syncthreads();
  float lsum = 0.f;
  for (int c = cl; c < nch; c += NCL) {
    const float mm = m_s[c][j];
    const float w = mm == -INFINITY ? 0.f : exp2f(mm - M_s[j]);
    lsum += w_s[c][j] * w;
    w_s[c][j] = w;
  }
  __syncthreads();
  red[cl][j] = lsum;
  __syncthreads();
  if (tid < kQRows) {
    float L = 0.f;
    for (int r = 0; r < NCL; ++r) L += red[r][tid];
    invL_s[tid] = 1.0f / L;
  }
  __syncthreads();

  // float4 f = (dt, q, row): row f % 16, dims 16*(f/64) + 4*((f/16)%4) .. +3.
  const int row = f % kQRows;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMergeBatch; ++c)
    if (c < nch) acc += w_s[c][row] * v[c];
  for (int c0 = kMergeBatch; c0 < nch; c0 += kMergeBatch) {
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      v[c] = c0 + c < nch ? src[(c0 + c) * cstride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMergeBatch; ++c)
      if (c0 + c < nch) acc += w_s[c0 + c][row] * v[c];
  }
  const int dim = 16 * (f / (4 * kQRows)) + 4 * ((f / kQRows) % 4);
  const f32x4 res = acc * invL_s[row];
  if (a.out_hilo) {
    store_hilo4(reinterpret_cast<bf16*>(a.out),
                hilo_off(tile * kQRows + row, h * D + dim, a.n_q * D / 32), res);
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) +
                              swz_off(tile * kQRows + row, h * D + dim, a.n_q * D / 16, 4)) = res;
  }
}

// ------------------------------------------------------------------------------------------
// Launch
// ------------------------------------------------------------------------------------------
template <int D, int RPR>
static void launch_partial_bf16(int G, dim3 grid, const AttnArgs& a, hipStream_t stream) {
  switch (G) {
    case 1: attn_partial_bf16<D, 1, RPR><<<grid, 1 * kWave, 0, stream>>>(a); break;
    case 2: attn_partial_bf16<D, 2, RPR><<<grid, 2 * kWave, 0, stream>>>(a); break;
    case 4: attn_partial_lds<D, 4, RPR><<<grid, 4 * kWave, 0, stream>>>(a); break;
    case 8: attn_partial_lds<D, 8, RPR><<<grid, 8 * kWave, 0, stream>>>(a); break;
    default: break;
  }
}

static hipError_t launch_partial(int bf16_dtype, const AttnArgs& a, int tiles,
                                 hipStream_t stream) {
  dim3 grid(a.nc, a.n_kv, tiles);
  const int G = a.n_q / a.n_kv;
  if (!block_attention_supported(bf16_dtype, a.head_dim, G)) return hipErrorInvalidValue;
  if (bf16_dtype) {
    if (a.head_dim == 128) {
      if (a.rpr == 32) launch_partial_bf16<128, 32>(G, grid, a, stream);
      else launch_partial_bf16<128, 16>(G, grid, a, stream);
    } else {
      if (a.rpr == 32) launch_partial_bf16<64, 32>(G, grid, a, stream);
      else launch_partial_bf16<64, 16>(G, grid, a, stream);
    }
  } else {
    const int R = G * kQRows;
    if (a.head_dim == 128) {
      if (R == 32) attn_partial_f32<128, 32><<<grid, kThreads, 0, stream>>>(a);
      else attn_partial_f32<128, 64><<<grid, kThreads, 0, stream>>>(a);
    } else {
      if (R == 32) attn_partial_f32<64, 32><<<grid, kThreads, 0, stream>>>(a);
      else if (R == 64) attn_partial_f32<64, 64><<<grid, kThreads, 0, stream>>>(a);
      else attn_partial_f32<64, 128><<<grid, kThreads, 0, stream>>>(a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_block_attention(int bf16_dtype, const AttnArgs& a, int tiles,
                                  hipStream_t stream) {
  if (a.nc < 1 || a.nc > kAttnMaxChunks || a.chunk < 32 || a.chunk % 32 ||
      a.chunk > kAttnMaxChunkKeys)
    return hipErrorInvalidValue;
  if ((a.rpr != 16 && a.rpr != 32) || a.nbk < 1 || a.nbk > a.rpr || tiles % (a.rpr / 16))
    return hipErrorInvalidValue;
  hipError_t e = launch_partial(bf16_dtype, a, tiles, stream);
  if (e != hipSuccess) return e;
  dim3 grid(a.n_q, a.head_dim / 32, tiles);
  constexpr int kSmallNc = 16;
  if (a.head_dim == 128) {
    if (a.nc <= kSmallNc) attn_merge<128, kSmallNc><<<grid, kMergeThreads, 0, stream>>>(a);
    else attn_merge<128, kAttnMaxChunks><<<grid, kMergeThreads, 0, stream>>>(a);
  } else {
    if (a.nc <= kSmallNc) attn_merge<64, kSmallNc><<<grid, kMergeThreads, 0, stream>>>(a);
    else attn_merge<64, kAttnMaxChunks><<<grid, kMergeThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

bool block_attention_supported(int bf16_dtype, int head_dim, int group) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (bf16_dtype) return group == 1 || group == 2 || group == 4 || group == 8;
  // fp32 VALU kernel: 32..128 query rows per group, LDS-bounded at d = 128.
  if (group != 2 && group != 4 && group != 8) return false;
  return !(head_dim == 128 && group == 8);
}

}  // namespace dflash
