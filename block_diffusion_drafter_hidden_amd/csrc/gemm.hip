// Weight-streaming GEMM for the DFlash drafter: out = A . W^T with a fused epilogue.
//
// Every drafter GEMM has few rows (16 block slots per request, or the injected context rows)
// and a large weight matrix, so at small batch the kernel's job is to stream the packed bf16
// weights from HBM at full bandwidth and feed each 16-byte lane chunk straight into a 16x16
// MFMA step.  Weights are bf16 (or fp32 for fp32 models); activations are fp32 in memory
// and enter a bf16 MFMA as a sum of bf16 pieces (see AFrag), except the bf16 target
// features of the fusion GEMM, which are exact in one piece.  (The LM head once took only
// the leading piece of its input at many rows; its logits then erred by up to 2.1e-2 at the
// 8B shapes, past half the 2e-2 band within which a drafted id may differ, so every kernel
// now multiplies both pieces.)  Activations the drafter produces itself live in the
// fragment layout (swz_off), so a wave's A operand for one k-tile is a couple of fully
// coalesced 1 KB reads; the epilogues write their outputs in that layout for the next GEMM.
//
// Work split.  A wave owns NPW consecutive n-tiles (16 output columns each) and a slice of
// the k range; the `ksub` waves of a tile group cover the whole k range and are reduced
// through LDS in wave order, so a workgroup produces complete outputs and no workgroup
// ever waits on another.  RMSNorm of the input is folded in: the kernel that produces the
// residual stream also writes x * gamma of the next norm and per-n-tile partial sums of
// squares; the normed GEMM streams x * gamma like any activation and scales each finished
// row by 1/sqrt(sum / K + eps) before the epilogue.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace dflash {

constexpr int kMaxWaves = kMaxGemmThreads / kWave;
constexpr int kXcds = 8;               // accelerator complex dies (one L2 each)
constexpr int kRedSlots = 16;          // waves * NPW * MT <= 16 (checked on the host)
constexpr int kTileFloats = 64 * 65;   // (MT*16) * (cols + 1) <= 4160 (checked on the host)

struct GemmSmem {
  f32x4 red[kRedSlots][kWave];
  float tile[kTileFloats];
  float ss_flat[kMaxWaves * kWave];   // per-thread partial sums of squares
  float rstd[64];
};

// Weight loads are non-temporal: every weight byte is read once per call, so they should not
// displace the activations the other workgroups re-read from L2 (measured 7-12% faster).
__device__ inline i32x4 load16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// ------------------------------------------------------------------------------------------
// Epilogues on the workgroup's dense fp32 tile: rows MT*16, columns cols (tile-major).
// ------------------------------------------------------------------------------------------
// Residual values (and gains) a thread uses in the epilogue, read at kernel start so the
// epilogue has no dependent global load: iteration i of the epilogue loop uses element i.
template <int MT, int NPW>
struct ResidualPrefetch {
  static constexpr int kN = 4 * NPW * MT <= 8 ? 4 * NPW * MT : 0;   // per thread, ksub = 1 bound
};
// The prefetched values of a thread's first N epilogue elements: residual x and the next
// RMSNorm's gain of the element's column.
template <int N>
struct EpiPrefetch {
  float x[N > 0 ? N : 1];
  float g[N > 0 ? N : 1];
};

// Per-row position and cache page of the Q|K|V and injection epilogues, looked up once per
// row into LDS (not by every pair of the row): by the epilogue itself, or, in the streaming
// kernel, at kernel start so the lookups' latency hides under the main loop.
constexpr int kEpiRows = 128;
__device__ inline int* epi_row_pos() {
  __shared__ int buf[kEpiRows];
  return buf;
}
__device__ inline int* epi_row_page() {
  __shared__ int buf[kEpiRows];
  return buf;
}
template <int EPI>
__device__ inline void epi_rows_fill(const GemmParams& p, int m0, int rows) {
  int* row_pos = epi_row_pos();
  int* row_page = epi_row_page();
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    const int m = m0 + r;
    int position = 0, page = 0;
    if (m < p.M) {
      if constexpr (EPI == EPI_QKV) {
        position = p.ctx_lens[m / p.rpr] + m % p.rpr;
        if (p.k_pool && m < p.kv_rows) page = p.block_table[position / kPage];
      } else {
        position = p.pos[m];
        page = p.block_table[(long long)p.seq_idx[m] * p.max_pages + position / kPage];
      }
    }
    row_pos[r] = position;
    row_page[r] = page;
  }
}

// `part`: the workgroup's column-block index (the argmax partial it writes).  SG: n-tiles per
// partial sum of squares of the residual epilogue (1: one per n-tile, the streaming kernel;
// kTallNT: one per 128-column block, the 128-row kernel).
template <typename T, int MT, int EPI, int NPRE, int SG = 1, bool kRowsFilled = false>
__device__ void run_epilogue(const GemmParams& p, float* tl, int cols, int tile0, int mblock,
                             int z, int part, const EpiPrefetch<NPRE>& pre) {
  const int rows = MT * 16;
  const int ld = cols + 1;
  const int m0 = mblock * rows;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;

  constexpr int kPer = Elem<T>::kPerLane;
  const int kto = p.ldo / (4 * kPer);   // k-tiles of the output as the next GEMM's A
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESIDUAL) {
    // Element idx of the tile; `xp` and `gp` are its prefetched residual value and gain when
    // known.
    auto store = [&](int idx, const float* xp, const float* gp) {
      const int r = idx / cols, c = idx % cols;
      const int m = m0 + r;
      if (m >= p.M) return;
      const long long off = swz_off(m, tile0 * 16 + c, kto, kPer);
      float* o = reinterpret_cast<float*>(p.out) + off;
      if constexpr (EPI == EPI_STORE) {
        *o = tl[r * ld + c];
      } else {
        const float v = (xp ? *xp : *o) + tl[r * ld + c];
        *o = v;
        if (p.xg_out) {
          const float xg = v * (gp ? *gp : p.gamma_next[tile0 * 16 + c]);
          if constexpr (std::is_same<T, bf16>::value)
            store_hilo(reinterpret_cast<bf16*>(p.xg_out), hilo_off(m, tile0 * 16 + c, kto), xg);
          else
            reinterpret_cast<float*>(p.xg_out)[off] = xg;
          tl[r * ld + c] = v;   // kept for the sums of squares below
        }
      }
    };
    int idx0 = tid;
    if constexpr (NPRE > 0) {   // iterations covered by the prefetch (static indices)
#pragma unroll
      for (int i = 0; i < NPRE; ++i)
        if (tid + i * nthr < rows * cols) store(tid + i * nthr, &pre.x[i], &pre.g[i]);
      idx0 = tid + NPRE * nthr;
    }
    for (int idx = idx0; idx < rows * cols; idx += nthr) store(idx, nullptr, nullptr);
    if constexpr (EPI == EPI_RESIDUAL && SG > 1) {
      if (p.xg_out) {   // one partial sum of squares per row over the whole column block
        __syncthreads();
        for (int r = tid; r < rows; r += nthr) {
          const int m = m0 + r;
          if (m >= p.M) continue;
          float ss = 0.f;
          for (int c = 0; c < cols; ++c) {
            const float v = tl[r * ld + c];
            ss += v * v;
          }
          p.ssq_out[(long long)(tile0 / SG) * p.ssq_ld + m] = ss;
        }
      }
    } else if constexpr (EPI == EPI_RESIDUAL) {
      if (p.xg_out) {   // partial sum of squares of every row over each n-tile's 16 columns
        __syncthreads();
        const int ntl = cols / 16;
        for (int idx = tid; idx < rows * ntl; idx += nthr) {
          const int r = idx % rows, jt = idx / rows;
          const int m = m0 + r;
          if (m >= p.M) continue;
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const float v = tl[r * ld + jt * 16 + c];
            ss += v * v;
          }
          p.ssq_out[(long long)(tile0 + jt) * p.ssq_ld + m] = ss;
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU && std::is_same<T, bf16>::value) {
    // Thread: the 8 outputs of one n-tile for one row -- one lane fragment of the pair
    // layout, stored as two 16-byte pieces (hi, lo); consecutive threads take consecutive
    // rows, i.e. consecutive fragments.
    const int ntl = cols / 16;
    for (int idx = tid; idx < rows * ntl; idx += nthr) {
      const int r = idx % rows, jt = idx / rows;
      const int m = m0 + r;
      if (m >= p.M) continue;
      const float* g = tl + r * ld + jt * 16;
      float h[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) h[c] = silu(g[c]) * g[8 + c];
      int hi[4], lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        hi[u] = bf16_pair_split(h[2 * u], h[2 * u + 1]);
        lo[u] = bf16_pair(h[2 * u], h[2 * u + 1]);
      }
      bf16* dst = reinterpret_cast<bf16*>(p.out) + hilo_off(m, (tile0 + jt) * 8, kto);
      *reinterpret_cast<i32x4*>(dst) = i32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<i32x4*>(dst + kHiLoStride) = i32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int half_cols = cols / 2;
    for (int idx = tid; idx < rows * half_cols; idx += nthr) {
      const int r = idx / half_cols, q = idx % half_cols;
      const int jt = q / 8, c = q % 8;  // tile within the workgroup, gate column
      const int m = m0 + r;
      if (m >= p.M) continue;
      const float gate = tl[r * ld + jt * 16 + c];
      const float up = tl[r * ld + jt * 16 + 8 + c];
      const float h = silu(gate) * up;
      if constexpr (std::is_same<T, bf16>::value)
        store_hilo(reinterpret_cast<bf16*>(p.out), hilo_off(m, (tile0 + jt) * 8 + c, kto), h);
      else
        reinterpret_cast<float*>(p.out)[swz_off(m, (tile0 + jt) * 8 + c, kto, kPer)] = h;
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    static_assert(MT * 16 <= kEpiRows, "rows of an epilogue tile");
    if constexpr (!kRowsFilled) {
      epi_rows_fill<EPI>(p, m0, rows);
      __syncthreads();
    }
    const int* row_pos = epi_row_pos();
    const int* row_page = epi_row_page();
    const int d = p.head_dim, half = d / 2, tph = d / 16;
    const int pairs = cols / 2;
    for (int idx = tid; idx < rows * pairs; idx += nthr) {
      const int r = idx / pairs, q = idx % pairs;
      const int jt = q / 8, pp = q % 8;
      const int m = m0 + r;
      if (m >= p.M) continue;
      const int j = tile0 + jt;  // n-tile within the launch
      const int head = j / tph, t = j % tph;
      float a0 = tl[r * ld + jt * 16 + 2 * pp], a1 = tl[r * ld + jt * 16 + 2 * pp + 1];
      const bool rope = EPI == EPI_QKV ? head < p.n_q + p.n_kv : head < p.n_kv;
      int d0, d1;  // head dims of the two columns
      const int position = row_pos[r];
      if (rope) {
        const int i = 8 * t + pp;
        float cs, sn;
        rope_cos_sin(position, p.inv_freq[i], &cs, &sn);
        const float y0 = a0 * cs - a1 * sn, y1 = a1 * cs + a0 * sn;
        a0 = y0;
        a1 = y1;
        d0 = i;
        d1 = i + half;
      } else {
        d0 = 16 * t + 2 * pp;
        d1 = d0 + 1;
      }
      if constexpr (EPI == EPI_QKV) {
        const int rpr = p.rpr, b = m / rpr, slot = m % rpr;
        if (head < p.n_q) {
          float* dst = p.q_out + ((long long)m * p.n_q + head) * d;
          dst[d0] = a0;
          dst[d1] = a1;
        } else {
          const bool is_k = head < p.n_q + p.n_kv;
          const int h = is_k ? head - p.n_q : head - p.n_q - p.n_kv;
          if (p.k_pool) {   // input-fusion prefill: the cache takes the row, and the block
                            // keys/values the stored (rounded) value
            a0 = Elem<T>::to_f(Elem<T>::from_f(a0));
            a1 = Elem<T>::to_f(Elem<T>::from_f(a1));
            if (m < p.kv_rows) {
              const long long page = row_page[r];
              const int ps = position % kPage;
              if (is_k) {
                T* dst = reinterpret_cast<T*>(p.k_pool) + ((page * p.n_kv + h) * kPage + ps) * d;
                dst[d0] = Elem<T>::from_f(a0);
                dst[d1] = Elem<T>::from_f(a1);
              } else {
                T* dst = reinterpret_cast<T*>(p.v_pool) + (page * p.n_kv + h) * d * kPage + ps;
                dst[d0 * kPage] = Elem<T>::from_f(a0);
                dst[d1 * kPage] = Elem<T>::from_f(a1);
              }
            }
          }
          if (is_k) {
            float* dst = p.bk_out + (((long long)b * p.n_kv + h) * rpr + slot) * d;
            dst[d0] = a0;
            dst[d1] = a1;
          } else {
            float* dst = p.bv_out + ((long long)b * p.n_kv + h) * d * rpr;
            dst[d0 * rpr + slot] = a0;
            dst[d1 * rpr + slot] = a1;
          }
        }
      } else {
        const int page = row_page[r];
        const int slot = position % kPage;
        const int h = rope ? head : head - p.n_kv;
        if (rope) {   // K page: [16 slots][d]
          T* dst = reinterpret_cast<T*>(p.k_pool) + (long long)z * p.pool_layer_elems +
                   (((long long)page * p.n_kv + h) * kPage + slot) * d;
          dst[d0] = Elem<T>::from_f(a0);
          dst[d1] = Elem<T>::from_f(a1);
        } else {      // V page, transposed: [d][16 slots]
          T* dst = reinterpret_cast<T*>(p.v_pool) + (long long)z * p.pool_layer_elems +
                   ((long long)page * p.n_kv + h) * d * kPage + slot;
          dst[d0 * kPage] = Elem<T>::from_f(a0);
          dst[d1 * kPage] = Elem<T>::from_f(a1);
        }
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    if (p.logits_out) {
      for (int idx = tid; idx < rows * cols; idx += nthr) {
        const int r = idx / cols, c = idx % cols;
        const int m = m0 + r;
        if (m >= p.M) continue;
        const long long orow = p.draft_rpr ? draft_out_row(m, p.draft_rpr, p.draft_nb) : m;
        if (orow < 0) continue;
        p.logits_out[orow * p.ldo + tile0 * 16 + c] = tl[r * ld + c];
      }
    }
    // One wave per row: lanes scan columns, then a wave-wide (value, index) maximum, stored
    // as this workgroup's part of the row (with keys2: the best two).
    const int lane = tid % kWave, wave = tid / kWave, nw = nthr / kWave;
    for (int r = wave; r < rows; r += nw) {
      const int m = m0 + r;
      if (m >= p.M) continue;
      unsigned long long best = 0, second = 0;
      for (int c = lane; c < cols; c += kWave) {
        const unsigned long long k = argmax_key(tl[r * ld + c], tile0 * 16 + c);
        top2_push(best, second, k);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long o1 = __shfl_xor(best, o, kWave);
        const unsigned long long o2 = __shfl_xor(second, o, kWave);
        top2_merge(best, second, o1, o2);
      }
      if (lane == 0) {
        p.keys[(long long)part * p.keys_ld + m] = best;
        if (p.keys2) p.keys2[(long long)part * p.keys_ld + m] = second;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Main kernel
// ------------------------------------------------------------------------------------------
// 16-byte A chunks per lane per k-tile and m-tile: the hi and lo pieces of the pair layout;
// one chunk of bf16 features; kPer / 4 chunks of fp32 values.
template <typename T, int AK> constexpr int kAChunks =
    AK == A_HILO ? 2 : (AK == A_ROW_BF16 ? 1 : Elem<T>::kPerLane / 4);
// Loads in flight per wave: a ring of R groups of KU k-tiles.  A group holds NPW weight
// chunks and MT * kAChunks activation chunks per k-tile; the ring is sized to about 96
// VGPRs (measured at one request: 2 x 3 k-tiles for Q|K|V, 2 x 4 for O / down, 2 x 2 for
// the LM head streamed as fast as 4-deep unrolled batches or faster).
template <typename T, int AK, int MT, int NPW> struct Ring {
  static constexpr int kUnits = NPW + MT * kAChunks<T, AK>;
  static constexpr int kTiles = 24 / kUnits < 2 ? 2 : (24 / kUnits > 8 ? 8 : 24 / kUnits);
  static constexpr int KU = kTiles >= 4 ? 2 : 1;
  static constexpr int R = kTiles / KU;
};

template <typename T, int AK, int MT, int NPW, int EPI, bool NORM>
__global__ __launch_bounds__(NPW >= 8 ? 256 : kMaxGemmThreads) void gemm_stream(GemmParams p) {
  __shared__ GemmSmem sm;
  constexpr int kTerms = EPI == EPI_INJECT ? 3 : 2;
  static_assert(AK != A_HILO || std::is_same<T, bf16>::value, "pair pieces feed bf16 MFMAs");
  typedef typename std::conditional<AK == A_ROW_BF16 || AK == A_HILO, bf16, float>::type AT;
  typedef AFrag<T, float, kTerms> FFrag;
  constexpr int kPer = Elem<T>::kPerLane;
  constexpr int NA = kAChunks<T, AK>;
  constexpr int KU = Ring<T, AK, MT, NPW>::KU, R = Ring<T, AK, MT, NPW>::R;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int ksub = p.ksub;
  const int tg = wave / ksub, ks = wave % ksub;
  // Workgroup -> (tile group, m-block).  With several m-blocks every weight tile is needed by
  // n_mblocks workgroups: workgroups are dispatched round-robin over the 8 XCDs, so the
  // m-blocks of one tile group are given ids that land on the same XCD back to back and the
  // repeated weight reads hit that XCD's L2 instead of HBM.
  int group, mblock;
  {
    const int L = blockIdx.x, nm = p.n_mblocks;
    const int n_groups = p.n_tiles / (p.tgpw * NPW);
    if (nm == 1) {
      group = L;
      mblock = 0;
    } else if (n_groups % kXcds == 0) {
      const int xcd = L % kXcds, slot = L / kXcds;
      group = (slot / nm) * kXcds + xcd;
      mblock = slot % nm;
    } else {
      group = L / nm;
      mblock = L % nm;
    }
  }
  const int wg_tile0 = group * p.tgpw * NPW;
  const int tile0 = wg_tile0 + tg * NPW;
  const int z = blockIdx.z;
  if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) epi_rows_fill<EPI>(p, mblock * MT * 16, MT * 16);
  // k-tiles of this wave: kb + i * kstep for i < nk.
  const int kw = (p.KT + ksub - 1) / ksub;
  const int kstep = p.kinter ? ksub : 1;
  const int kb = p.kinter ? ks : min(ks * kw, p.KT);
  const int ke = p.kinter ? p.KT : min(kb + kw, p.KT);
  const int nk = ke > kb ? (ke - kb + kstep - 1) / kstep : 0;
  const int G = (nk + KU - 1) / KU;   // groups of KU k-tiles
  // LM head: the workgroups of one XCD (dispatch goes round-robin over the 8) start their k
  // ranges at different k-tiles, so they do not all ask L2 for the same activation lines at
  // once (measured on the batch-1 draft pass: 192.5 -> 189 us).  Each wave still multiplies
  // every k-tile of its range once, in a rotated order.  The other GEMMs keep the plain
  // order (their gain was under 1 us, and their results then depend on the k-split alone,
  // not on how a call's rows are grouped).
  int krot = 0;
  if constexpr (EPI == EPI_ARGMAX) krot = nk > 0 ? (int)(((unsigned)group >> 3) * 5u % (unsigned)nk) : 0;

  const char* wp[NPW];
#pragma unroll
  for (int t = 0; t < NPW; ++t)
    wp[t] = p.W + (long long)z * p.w_zstride +
            (long long)(p.nt0 + tile0 + t) * p.nt_stride * kTileBytes + lane * 16;
  const long long kbytes = p.kt_stride * kTileBytes;

  // A pointers per m-tile.  Row-major kinds: this lane's row and k-slice; fragment layouts:
  // this lane's 16 bytes of k-tile 0.  M-tiles past the valid rows re-read the last valid
  // one (their rows reach only output rows the epilogue never stores, and a row of the
  // product depends on that row of A alone), so every load is in bounds and unconditional.
  constexpr int kGroups = kPer / 4;
  const AT* A = reinterpret_cast<const AT*>(p.A);
  const AT* arow[MT];
  const int n_mtiles_valid = (p.M + 15) / 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int mtile = min(mblock * MT + mt, n_mtiles_valid - 1);
    const int r = min(mtile * 16 + (lane & 15), p.M - 1);
    if constexpr (AK == A_SWZ)
      arow[mt] = A + (long long)mtile * p.KT * kGroups * 256 + lane * 4;
    else if constexpr (AK == A_HILO)
      arow[mt] = A + (long long)mtile * p.KT * 1024 + lane * 8;
    else
      arow[mt] = A + (long long)r * p.lda + (lane >> 4) * kPer;
  }

  struct Group {
    i32x4 w[KU][NPW];
    i32x4 a[KU][MT][NA];
  };
  Group ring[R];
  // Loads of group g; k-tiles past the wave's last re-read it (never out of bounds).
  auto load = [&](Group& gr, int g) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      int ki = min(g * KU + u, nk - 1) + krot;
      if (ki >= nk) ki -= nk;
      const int kt = kb + ki * kstep;
#pragma unroll
      for (int t = 0; t < NPW; ++t) gr.w[u][t] = load16(wp[t] + (long long)kt * kbytes);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (AK == A_HILO) {
          const AT* src = arow[mt] + (long long)kt * 1024;
          gr.a[u][mt][0] = *reinterpret_cast<const i32x4*>(src);
          gr.a[u][mt][1] = *reinterpret_cast<const i32x4*>(src + kHiLoStride);
        } else if constexpr (AK == A_ROW_BF16) {
          gr.a[u][mt][0] =
              *reinterpret_cast<const i32x4*>(arow[mt] + (long long)kt * Elem<T>::kTile);
        } else if constexpr (AK == A_SWZ) {
#pragma unroll
          for (int q = 0; q < NA; ++q)
            gr.a[u][mt][q] = *reinterpret_cast<const i32x4*>(
                arow[mt] + ((long long)kt * kGroups + q) * 256);
        } else {
#pragma unroll
          for (int q = 0; q < NA; ++q)
            gr.a[u][mt][q] = *reinterpret_cast<const i32x4*>(
                arow[mt] + (long long)kt * Elem<T>::kTile + 4 * q);
        }
      }
    }
  };
  // acc takes the products of the first A piece, acc_lo those of the others: two
  // independent MFMA chains per tile (added together after the loop).
  f32x4 acc[NPW][MT], acc_lo[NPW][MT];
#pragma unroll
  for (int t = 0; t < NPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = acc_lo[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // MFMAs of group g; with `check`, k-tiles past the wave's last are skipped (wave-uniform).
  auto compute = [&](const Group& gr, int g, bool check) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (check && g * KU + u >= nk) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (AK == A_HILO) {   // ready-made pieces: hi feeds acc, lo feeds acc_lo
#pragma unroll
          for (int t = 0; t < NPW; ++t) {
            acc[t][mt] = mfma_tile<T>(gr.a[u][mt][0], gr.w[u][t], acc[t][mt]);
            acc_lo[t][mt] = mfma_tile<T>(gr.a[u][mt][1], gr.w[u][t], acc_lo[t][mt]);
          }
        } else if constexpr (AK == A_ROW_BF16) {   // bf16 features: exact in one piece
#pragma unroll
          for (int t = 0; t < NPW; ++t)
            acc[t][mt] = mfma_tile<T>(gr.a[u][mt][0], gr.w[u][t], acc[t][mt]);
        } else {   // fp32 values: split into pieces right before their MFMAs
          float f[kPer];
#pragma unroll
          for (int q = 0; q < NA; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * q + e] = __int_as_float(gr.a[u][mt][q][e]);
          FFrag a;
          a.from_floats(f);
#pragma unroll
          for (int t = 0; t < NPW; ++t)
#pragma unroll
            for (int q = 0; q < FFrag::kTerms; ++q)
              if (q == 0) acc[t][mt] = mfma_tile<T>(a.part[q], gr.w[u][t], acc[t][mt]);
              else acc_lo[t][mt] = mfma_tile<T>(a.part[q], gr.w[u][t], acc_lo[t][mt]);
        }
      }
    }
  };

  // The ring's first loads go out before anything else, so the first weights arrive as
  // early as possible; the values only the epilogue needs are fetched after them.
  if (nk > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) load(ring[r], r);
  }
  // RMSNorm: this thread's share of the rows' partial sums of squares, summed after the
  // main loop.  Thread t always serves row t % rows (blockDim is a multiple of 64, rows =
  // 16 * MT <= 64).
  constexpr int kSsqPer = NORM ? 16 : 1;
  float sq[kSsqPer];
  if constexpr (NORM) {
    const int rows = MT * 16, total = rows * p.ssq_parts;
    const int m = mblock * rows + threadIdx.x % rows;
#pragma unroll
    for (int i = 0; i < kSsqPer; ++i) {
      const int idx = threadIdx.x + i * blockDim.x;
      sq[i] = idx < total && m < p.M ? p.ssq_in[(long long)(idx / rows) * p.ssq_ld + m] : 0.f;
    }
  }
  // Residual values a thread adds in the epilogue (read now, so the epilogue has no
  // dependent global load).
  constexpr int NPRE = EPI == EPI_RESIDUAL ? ResidualPrefetch<MT, NPW>::kN : 0;
  EpiPrefetch<NPRE> pre;
  if constexpr (NPRE > 0) {
    const int rows = MT * 16, cols = p.tgpw * NPW * 16;
    const int kto = p.ldo / (4 * kPer);
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int idx = threadIdx.x + i * blockDim.x;
      const int m = mblock * rows + idx / cols;
      const bool ok = idx < rows * cols && m < p.M;
      pre.x[i] = ok ? reinterpret_cast<const float*>(p.out)[swz_off(m, wg_tile0 * 16 + idx % cols,
                                                                   kto, kPer)]
                    : 0.f;
      pre.g[i] = ok && p.xg_out ? p.gamma_next[wg_tile0 * 16 + idx % cols] : 0.f;
    }
  }

  // Main loop: group g is multiplied while groups g + 1 .. g + R - 1 are in flight, then its
  // registers are refilled with group g + R.  Full rounds of R groups whose refills are all
  // needed run without conditions; the last groups follow.
  if (nk > 0) {
    int g = 0;
    for (; g + 2 * R <= G; g += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        compute(ring[r], g + r, false);
        load(ring[r], g + r + R);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (g + r < G) {
        compute(ring[r], g + r, true);
        if (g + r + R < G) load(ring[r], g + r + R);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (g + R + r < G) compute(ring[r], g + R + r, true);
  }

#pragma unroll
  for (int t = 0; t < NPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] += acc_lo[t][mt];

  // k-slices of a tile group: park slices 1.., add them to slice 0 in wave order.
  if (ksub > 1 && ks > 0) {
#pragma unroll
    for (int t = 0; t < NPW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sm.red[(wave * NPW + t) * MT + mt][lane] = acc[t][mt];
  }
  if constexpr (NORM) {   // per-thread sums of the prefetched partials (in part order)
    const int rows = MT * 16, total = rows * p.ssq_parts;
    const int m = mblock * rows + threadIdx.x % rows;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kSsqPer; ++i) s += sq[i];
    for (int idx = threadIdx.x + kSsqPer * blockDim.x; idx < total; idx += blockDim.x)
      if (m < p.M) s += p.ssq_in[(long long)(idx / rows) * p.ssq_ld + m];
    sm.ss_flat[threadIdx.x] = s;
  }
  __syncthreads();
  if (ksub > 1 && ks == 0) {
    for (int q = 1; q < ksub; ++q)
#pragma unroll
      for (int t = 0; t < NPW; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += sm.red[((wave + q) * NPW + t) * MT + mt][lane];
  }
  if constexpr (NORM) {
    const int rows = MT * 16;
    if (threadIdx.x < rows) {
      float s = 0.f;
      for (int j = threadIdx.x; j < (int)blockDim.x; j += rows) s += sm.ss_flat[j];
      sm.rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)(p.KT * Elem<T>::kTile) + p.eps);
    }
    __syncthreads();
  }
  const int cols = p.tgpw * NPW * 16;
  const int ld = cols + 1;
  if (ks == 0) {
#pragma unroll
    for (int t = 0; t < NPW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = mt * 16 + (lane >> 4) * 4 + j;
          float v = acc[t][mt][j];
          if constexpr (NORM) v *= sm.rstd[r];
          sm.tile[r * ld + (tg * NPW + t) * 16 + (lane & 15)] = v;
        }
  }
  __syncthreads();
  run_epilogue<T, MT, EPI, NPRE, 1, true>(p, sm.tile, cols, wg_tile0, mblock, z, group, pre);
}

// ------------------------------------------------------------------------------------------
// Tall variant for many rows (batched drafts, prefill chunks): a workgroup of 4 waves owns a
// 128-row x 128-column output block and walks K one 32-wide k-tile at a time.  Each k-tile's
// W block (8 n-tiles, 8 KB) is staged in LDS once (double-buffered, later k-tiles' loads in
// flight during this one's MFMAs).  Activations in the pair layout are MFMA fragments
// already: each wave loads the hi and lo fragments of its own 32 rows straight into
// registers and computes a 32 x 128 strip (2 x 8 tile products, each as hi + lo bf16 MFMAs).
// The other kinds (the injection's fp32 input, split into three pieces; the fusion's bf16
// rows) are staged in LDS with W, converted once per workgroup, and each wave computes a
// 64 x 64 quarter.  Weights are thus read once per 128 rows and activations once per 128
// columns.  The finished block goes through LDS to the same epilogues as the streaming
// kernel.
// ------------------------------------------------------------------------------------------
constexpr int kTallM = 128, kTallN = 128;
constexpr int kTallMT = kTallM / 16, kTallNT = kTallN / 16;
constexpr int kTallColRows = 4;   // row blocks up to which the order is column-block major

struct TallStage {
  i32x4 a[2][3][kTallMT][kWave];   // [buf][piece][m-tile][lane]: bf16 pieces of A fragments
  i32x4 w[2][kTallNT][kWave];      // [buf][n-tile][lane]: packed bf16 B fragments
};
union TallSmem {
  TallStage st;
  float tile[kTallM * (kTallN + 1)];
};

// RMSNorm of a 128-row block: the rows' sums of squares come as ssq_parts partials.  Thread
// t serves row t % 128 and parts t / 128 + 2 i: the first 8 of them are fetched early
// (tall_ssq_prefetch, so the loads overlap the main loop), the rest at the end; the two
// half sums of a row are added last (tall_rstd, which leaves 1 / rms in rstd_s).
__device__ inline void tall_ssq_prefetch(const GemmParams& p, int rb, float (&sq)[8]) {
  const int tid = threadIdx.x, m = rb * kTallM + tid % kTallM;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int part = tid / kTallM + 2 * i;
    sq[i] = part < p.ssq_parts && m < p.M ? p.ssq_in[(long long)part * p.ssq_ld + m] : 0.f;
  }
}
__device__ inline void tall_rstd(const GemmParams& p, int rb, const float (&sq)[8],
                                 float* ssq_s, float* rstd_s) {
  const int tid = threadIdx.x, m = rb * kTallM + tid % kTallM;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += sq[i];
  for (int part = tid / kTallM + 16; part < p.ssq_parts; part += 2)
    if (m < p.M) s += p.ssq_in[(long long)part * p.ssq_ld + m];
  ssq_s[tid] = s;
  __syncthreads();
  if (tid < kTallM)
    rstd_s[tid] = 1.0f / sqrtf((ssq_s[tid] + ssq_s[tid + kTallM]) / (float)(p.KT * 32) + p.eps);
  __syncthreads();
}

// k-split modes of the 128-row kernel: store / residual epilogues reduce row-major partials
// (ksplit_reduce_kernel); the Q|K|V epilogue reduces whole partial blocks
// (ksplit_tile_reduce_kernel) and then runs the unsplit epilogue.
template <int EPI> constexpr bool kRowSplit = EPI == EPI_RESIDUAL || EPI == EPI_STORE;
template <int EPI> constexpr bool kTileSplit = EPI == EPI_QKV;

template <int AK, int EPI, bool NORM>
__global__ __launch_bounds__(256, 2) void gemm_tall(GemmParams p) {
  __shared__ TallSmem sm;
  __shared__ float rstd_s[kTallM];
  __shared__ float ssq_s[256];
  static_assert(AK == A_HILO || AK == A_SWZ || AK == A_ROW_BF16, "activation kinds");
  // Staged kinds, bf16 pieces per A value: the bf16 target features are exact; the fp32
  // fused features split in three (the injection's results end in the cache).
  constexpr int kTerms = AK == A_ROW_BF16 ? 1 : 3;
  static_assert(AK != A_SWZ || EPI == EPI_INJECT, "fp32 fragments feed the injection");
  constexpr int kAChunks = AK == A_ROW_BF16 ? 2 : 4;   // 16-byte A chunks per thread
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;           // this wave's 64 x 64 quarter
  const int z = blockIdx.z;

  // Workgroup -> (column block, row block).  Up to kTallColRows row blocks: workgroups are
  // dealt round-robin to the 8 XCDs and the ids are arranged so that each XCD takes whole
  // column blocks, all their row blocks back to back -- a weight block comes from HBM once
  // and is re-read from that XCD's L2 (the grid is padded to whole rounds of 8 column
  // blocks; padding workgroups exit at once).  More row blocks: row-block major, so the
  // workgroups resident at one time share a row block whose activations stay in L2 while
  // the weights stream past (measured faster once the activations outgrow an XCD's L2).
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT, nrb = p.n_mblocks;
  int cb, rb;
  if (nrb <= kTallColRows) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    cb = (slot / nrb) * kXcds + xcd;
    rb = slot % nrb;
    if (cb >= ncb) return;
  } else {
    cb = blockIdx.x % ncb;
    rb = blockIdx.x / ncb;
  }
  // k-tiles [kb, kb + KT) of this workgroup's slice of the k range.
  const int S = (kRowSplit<EPI> || kTileSplit<EPI>) ? max(p.ksplit, 1) : 1;
  const int sl = blockIdx.y;
  const int kb = (sl * p.KT) / S;
  const int KT = ((sl + 1) * p.KT) / S - kb;
  const int ntv = min(kTallNT, p.n_tiles - cb * kTallNT);   // valid n-tiles (ragged last)
  const int mtile0 = rb * kTallMT;                   // first m-tile of the block
  const int n_mtiles_valid = (p.M + 15) / 16;
  const float* A = reinterpret_cast<const float*>(p.A);
  const char* W = p.W + (long long)z * p.w_zstride +
                  (long long)(p.nt0 + cb * kTallNT) * p.nt_stride * kTileBytes;

  // RMSNorm of this block's rows (unsplit: a k-split's reduction applies it).
  float sq[8];
  if constexpr (NORM) {
    if (S == 1) tall_ssq_prefetch(p, rb, sq);
  }

  // Staged kinds: global -> register staging of one k-tile, 4 (2) A chunks and 2 W chunks of
  // 16 bytes per thread.  A ring of kRing register stages keeps kRing - 1 k-tiles of loads
  // in flight beyond the one being multiplied (the three-piece split needs the registers
  // a deeper ring would take).
  constexpr int kRing = 2;
  f32x4 ra[kRing][kAChunks];
  i32x4 rw[kRing][2];
  // Loads are unconditional (no divergent branches, so the waits stay precise): k-tiles past
  // the end re-read the last one, and m-tiles past the rows re-read the last valid m-tile --
  // those rows only reach output rows the epilogue never stores.
  // A chunk c (16 bytes: 4 floats of one fragment lane) is m-tile c / 128, lane (c / 2) % 64,
  // half c % 2 of the lane's 8 k values, so neighbouring threads write neighbouring 8-byte
  // halves of the LDS fragments.
  // bf16 rows: chunk c is m-tile c / 64, lane c % 64 (row l % 16, k 8 (l / 16) .. + 8), read
  // from the row (rows past M re-read row M - 1).  n-tiles past a ragged last column block
  // re-read its last valid n-tile (their columns are never stored).
  auto load_stage = [&](int kt, f32x4 (&a)[kAChunks], i32x4 (&w)[2]) {
    const int ktc = kb + min(kt, KT - 1);
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + i * 256;
      if constexpr (AK == A_ROW_BF16) {
        const int l = c % 64, row = min((mtile0 + c / 64) * 16 + (l & 15), p.M - 1);
        a[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const bf16*>(p.A) +
                                               (long long)row * p.lda + ktc * 32 + (l >> 4) * 8);
        continue;
      }
      const int mt = c / 128;
      const int mtc = min(mtile0 + mt, n_mtiles_valid - 1);
      const int g = c % 2, l = (c / 2) % 64;
      a[i] = *reinterpret_cast<const f32x4*>(A + (((long long)mtc * p.KT + ktc) * 2 + g) * 256 +
                                             l * 4);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256, nt = min(c / 64, ntv - 1), l = c % 64;
      w[i] = load16(W + ((long long)nt * p.nt_stride + (long long)ktc * p.kt_stride) *
                            kTileBytes + l * 16);
    }
  };
  // The fp32 A values are split into their bf16 pieces here, once per workgroup, and the
  // pieces stored as MFMA fragments.
  auto store_stage = [&](int buf, const f32x4 (&a)[kAChunks], const i32x4 (&w)[2]) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + i * 256, mt = c / 128;
      if constexpr (AK == A_ROW_BF16) {
        sm.st.a[buf][0][c / 64][c % 64] = __builtin_bit_cast(i32x4, a[i]);
        continue;
      }
      const int g = c % 2, l = (c / 2) % 64;
      float f[4] = {a[i][0], a[i][1], a[i][2], a[i][3]};
#pragma unroll
      for (int t = 0; t < kTerms; ++t) {
        const int h01 = bf16_pair_split(f[0], f[1]), h23 = bf16_pair_split(f[2], f[3]);
        reinterpret_cast<i32x2*>(&sm.st.a[buf][t][mt][l])[g] = i32x2{h01, h23};
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      sm.st.w[buf][c / 64][c % 64] = w[i];
    }
  };

  // Wave tiles.  Staged kinds: 64 x 64 quarters (wm, wn).  Pair layout and fp32 fragments: a
  // 32-row x 128-column strip per wave (rows 32 wave .. + 32), so no two waves need the same
  // A fragment.
  constexpr bool kDirect = AK == A_HILO || AK == A_SWZ;
  constexpr int MI = kDirect ? 2 : 4, NJ = kDirect ? 8 : 4;
  const int row0 = kDirect ? wave * 32 : wm * 64, col0 = kDirect ? 0 : wn * 64;
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (kDirect) {
    // The pair layout already holds the MFMA A fragments: each wave loads its two m-tiles'
    // hi and lo fragments (1 KB each, coalesced) straight into registers, kR k-tiles ahead.
    // Only W is shared, so only W goes through LDS: 8 KB written and 32 KB read per k-tile
    // instead of 24 KB and 48 KB, with a third of the LDS instructions.
    // fp32 fragments (the injection's fused features): the lane's 8 values of a k-tile are
    // two 16-byte halves, split in registers into three bf16 pieces -- by every wave for its
    // own rows, instead of once per workgroup through LDS (measured: the LDS traffic of the
    // staged pieces had bound the 512-row injection).
    constexpr bool kSwz = AK == A_SWZ;
    const bf16* ap[2];
    const float* af32[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mtc = min(mtile0 + wave * 2 + i, n_mtiles_valid - 1);
      ap[i] = reinterpret_cast<const bf16*>(p.A) + (long long)mtc * p.KT * 1024 + lane * 8;
      af32[i] = A + (long long)mtc * p.KT * 512 + lane * 4;
    }
    constexpr int kR = 3;
    constexpr int kQ = kSwz ? 3 : 2;   // pieces per A value (hi and lo; three of an fp32)
    i32x4 da[kR][2][2], dw[kR][2];   // [stage][m-tile][piece or fp32 half], [stage][chunk]
    auto load_a = [&](int kt, i32x4 (&a)[2][2]) {
      const int ktc = kb + min(kt, KT - 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if constexpr (kSwz)
            a[i][q] = *reinterpret_cast<const i32x4*>(af32[i] + ((long long)ktc * 2 + q) * 256);
          else
            a[i][q] = *reinterpret_cast<const i32x4*>(ap[i] + (long long)ktc * 1024 +
                                                       q * kHiLoStride);
        }
    };
    auto load_w = [&](int kt, i32x4 (&w)[2]) {
      const int ktc = kb + min(kt, KT - 1);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256, nt = min(c / 64, ntv - 1), l = c % 64;
        w[i] = load16(W + ((long long)nt * p.nt_stride + (long long)ktc * p.kt_stride) *
                              kTileBytes + l * 16);
      }
    };
    auto store_w = [&](int buf, const i32x4 (&w)[2]) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256;
        sm.st.w[buf][c / 64][c % 64] = w[i];
      }
    };
    // Piece-major MFMA order: the products into one accumulator are 16 apart.
    auto compute = [&](int buf, const i32x4 (&a)[2][2]) {
      i32x4 wf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wf[j] = sm.st.w[buf][j][lane];
      i32x4 pc[2][kQ];   // the A pieces of the two m-tiles
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (kSwz) {   // values 0-3 from the first half, 4-7 from the second
          float f[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[e] = __int_as_float(a[i][0][e]);
            f[4 + e] = __int_as_float(a[i][1][e]);
          }
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            int h[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) h[u] = bf16_pair_split(f[2 * u], f[2 * u + 1]);
            pc[i][q] = i32x4{h[0], h[1], h[2], h[3]};
          }
        } else {
#pragma unroll
          for (int q = 0; q < kQ; ++q) pc[i][q] = a[i][q];
        }
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = mfma_tile<bf16>(pc[i][q], wf[j], acc[i][j]);
    };
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      load_w(r, dw[r]);
      load_a(r, da[r]);
    }
    store_w(0, dw[0]);
    __syncthreads();
    // Iteration kt: W stage kt % kR is in LDS and is refilled with k-tile kt + kR; A stage
    // kt % kR is multiplied, then refilled; W of k-tile kt + 1 moves to LDS.
    const int KTr = KT - KT % kR;
    for (int kt0 = 0; kt0 < KTr; kt0 += kR) {
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int kt = kt0 + r;
        load_w(kt + kR, dw[r]);
        compute(kt & 1, da[r]);
        load_a(kt + kR, da[r]);
        store_w((kt + 1) & 1, dw[(r + 1) % kR]);
        __syncthreads();
      }
    }
#pragma unroll
    for (int r = 0; r < kR - 1; ++r) {
      const int kt = KTr + r;
      if (kt < KT) {
        compute(kt & 1, da[r]);
        store_w((kt + 1) & 1, dw[(r + 1) % kR]);
        __syncthreads();
      }
    }
  } else {
  // One k-tile from LDS: every fragment read first (one wait), then the MFMAs ordered piece-
  // major so the two (three) products into one accumulator are 16 instructions apart.
  auto compute = [&](int buf) {
    i32x4 wf[4], af[kTerms][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wf[j] = sm.st.w[buf][wn * 4 + j][lane];
#pragma unroll
    for (int q = 0; q < kTerms; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) af[q][i] = sm.st.a[buf][q][wm * 4 + i][lane];
#pragma unroll
    for (int q = 0; q < kTerms; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_tile<bf16>(af[q][i], wf[j], acc[i][j]);
  };

  // Prologue: k-tiles 0 .. kRing-1 in flight, k-tile 0 in LDS buffer 0.
#pragma unroll
  for (int r = 0; r < kRing; ++r) load_stage(r, ra[r], rw[r]);
  store_stage(0, ra[0], rw[0]);
  __syncthreads();
  // Iteration kt: ring stage kt % kRing is free (its k-tile is in LDS) and is refilled with
  // k-tile kt + kRing; k-tile kt is multiplied from LDS; k-tile kt + 1 moves to LDS.
  // Full rounds of kRing k-tiles without conditions, then the remainder.
  const int KTr = KT - KT % kRing;
  for (int kt0 = 0; kt0 < KTr; kt0 += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int kt = kt0 + r;
      load_stage(kt + kRing, ra[r], rw[r]);
      compute(kt & 1);
      store_stage((kt + 1) & 1, ra[(r + 1) % kRing], rw[(r + 1) % kRing]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < kRing - 1; ++r) {
    const int kt = KTr + r;
    if (kt < KT) {
      compute(kt & 1);
      store_stage((kt + 1) & 1, ra[(r + 1) % kRing], rw[(r + 1) % kRing]);
      __syncthreads();
    }
  }
  }

  if constexpr (NORM) {
    if (S == 1) tall_rstd(p, rb, sq, ssq_s, rstd_s);
  }
  const int cols = ntv * 16, ld = cols + 1;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = row0 + i * 16 + (lane >> 4) * 4 + e;
        const int col = col0 + j * 16 + (lane & 15);
        float v = acc[i][j][e];
        if constexpr (NORM) {
          if (S == 1) v *= rstd_s[r];
        }
        if (col < cols) sm.tile[r * ld + col] = v;
      }
  __syncthreads();
  if (S > 1) {
    if constexpr (EPI == EPI_RESIDUAL) {
      // k-slice partial in the residual stream's fragment layout, [slice][offset of x]: 16-byte
      // pieces of 4 columns of one row, consecutive threads writing consecutive pieces, so
      // the reduction reads each slice as contiguously as it reads x (M and the block's
      // columns are multiples of 16 and 32 here).
      const int kto = p.ldo / 32, nkt = cols / 32;
      float* dst = p.partial + (long long)sl * p.M * p.ldo;
      for (int pc = tid; pc < kTallMT * nkt * 128; pc += 256) {
        const int ln = pc % 64, jb = (pc / 64) % 2, ktl = (pc / 128) % nkt, mtl = pc / 128 / nkt;
        const int r = mtl * 16 + (ln & 15), m = rb * kTallM + r;
        if (m >= p.M) continue;
        const float* t = sm.tile + r * ld + ktl * 32 + 8 * (ln >> 4) + 4 * jb;
        const f32x4 v = f32x4{t[0], t[1], t[2], t[3]};
        *reinterpret_cast<f32x4*>(
            dst + ((((long long)(m >> 4) * kto + cb * (kTallN / 32) + ktl) * 2 + jb) * 256 + ln * 4)) =
            v;
      }
    } else if constexpr (kRowSplit<EPI>) {   // k-slice partial, row-major [slice][row][column]
      const int quads = cols / 4;             // 16-byte stores of 4 columns
      for (int idx = tid; idx < kTallM * quads; idx += 256) {
        const int r = idx / quads, c = 4 * (idx % quads), m = rb * kTallM + r;
        if (m >= p.M) continue;
        const float* t = sm.tile + r * ld + c;
        *reinterpret_cast<f32x4*>(p.partial + ((long long)sl * p.M + m) * p.ldo + cb * kTallN +
                                  c) = f32x4{t[0], t[1], t[2], t[3]};
      }
    } else if constexpr (kTileSplit<EPI>) {   // whole block [slice][block][row][128 columns]
      const long long blk = (long long)rb * ncb + cb;
      float* dst = p.partial + ((long long)sl * ncb * nrb + blk) * (kTallM * kTallN);
      const int quads = cols / 4;
      for (int idx = tid; idx < kTallM * quads; idx += 256) {
        const int r = idx / quads, c = 4 * (idx % quads);
        if (rb * kTallM + r >= p.M) continue;
        const float* t = sm.tile + r * ld + c;
        *reinterpret_cast<f32x4*>(dst + r * kTallN + c) = f32x4{t[0], t[1], t[2], t[3]};
      }
    }
    return;
  }
  const EpiPrefetch<0> pre{};
  run_epilogue<bf16, kTallMT, EPI, 0, kTallNT>(p, sm.tile, cols, cb * kTallNT, rb, z, cb, pre);
}

// ------------------------------------------------------------------------------------------
// 256-row blocks for the LM head and gate|up over many rows: the 128-row kernel's W staging,
// but each of the 4 waves owns 64 rows (4 m-tiles) x the block's 128 columns, so the 8 KB of
// W a wave reads from LDS per k-tile feed 32 MFMAs per A piece instead of 16, and each W
// block read from HBM or L2 serves 256 rows.
//   EPI_ARGMAX, hi piece (refine mode): the block goes through a 128-row LDS tile in two
//   halves, two threads scan each row for its best three (value, index) keys and merge them
//   (measured against the in-register selection below: LM-head entry point at 480 rows
//   747 -> 694 us, at 1920 rows 2873 -> 2630 us).
//   EPI_ARGMAX, both pieces (logits out): in registers -- a lane scales its values by the
//   row's 1/rms, keeps the best two (value, index) keys of its column over the 8 n-tiles,
//   and the 16 lanes of a row group reduce with shuffles.
//   EPI_SWIGLU (hi + lo pieces): the finished block goes through a 128-row LDS tile in two
//   halves to the same epilogue as the 128-row kernel.
// ------------------------------------------------------------------------------------------
constexpr int kWideRows = 256, kWideMT = kWideRows / 16;

constexpr int kWideLd = kTallN + 4;   // row stride of the selection tile (16-byte rows)
union WideSmem {
  i32x4 w[2][kTallNT][kWave];          // [buf][n-tile][lane]: packed bf16 B fragments
  float tile[kTallM * kWideLd];        // epilogue tile: 128 rows of the block
};

// kQ: bf16 pieces of the input multiplied (2: hi and lo; 1: hi alone, the LM head's
// refine mode).
template <int EPI, int kQ>
__global__ __launch_bounds__(256, 2) void gemm_tall256(GemmParams p) {
  static_assert(EPI == EPI_ARGMAX || EPI == EPI_SWIGLU, "LM head and gate|up");
  static_assert(kQ == 2 || EPI == EPI_ARGMAX, "gate|up takes both pieces");
  __shared__ WideSmem sm;
  __shared__ float rstd_s[kWideRows];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT, nrb = (p.M + kWideRows - 1) / kWideRows;
  int cb, rb;   // same XCD-aware order as the 128-row kernel
  if (nrb <= kTallColRows) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    cb = (slot / nrb) * kXcds + xcd;
    rb = slot % nrb;
    if (cb >= ncb) return;
  } else {
    cb = blockIdx.x % ncb;
    rb = blockIdx.x / ncb;
  }
  const int KT = p.KT;
  const int ntv = min(kTallNT, p.n_tiles - cb * kTallNT);
  const int n_mtiles_valid = (p.M + 15) / 16;
  const char* W = p.W + (long long)(p.nt0 + cb * kTallNT) * p.nt_stride * kTileBytes;

  // RMSNorm: thread t serves row rb * 256 + t; its first 8 partials are fetched now.
  const int my_row = rb * kWideRows + tid;
  float sq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    sq[i] = i < p.ssq_parts && my_row < p.M ? p.ssq_in[(long long)i * p.ssq_ld + my_row] : 0.f;

  // This wave's 4 m-tiles (rows past M re-read the last valid m-tile; never stored).
  const bf16* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mtc = min(rb * kWideMT + wave * 4 + i, n_mtiles_valid - 1);
    ap[i] = reinterpret_cast<const bf16*>(p.A) + (long long)mtc * KT * 1024 + lane * 8;
  }
  constexpr int kR = 2;
  i32x4 da[kR][4][kQ], dw[kR][2];
  auto load_a = [&](int kt, i32x4 (&a)[4][kQ]) {
    const long long off = (long long)min(kt, KT - 1) * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < kQ; ++q)
        a[i][q] = *reinterpret_cast<const i32x4*>(ap[i] + off + q * kHiLoStride);
  };
  auto load_w = [&](int kt, i32x4 (&w)[2]) {
    const int ktc = min(kt, KT - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256, nt = min(c / 64, ntv - 1), l = c % 64;
      w[i] = load16(W + ((long long)nt * p.nt_stride + (long long)ktc * p.kt_stride) *
                            kTileBytes + l * 16);
    }
  };
  auto store_w = [&](int buf, const i32x4 (&w)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      sm.w[buf][c / 64][c % 64] = w[i];
    }
  };
  f32x4 acc[4][kTallNT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kTallNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const i32x4 (&a)[4][kQ]) {
#pragma unroll
    for (int j = 0; j < kTallNT; ++j) {
      const i32x4 wf = sm.w[buf][j][lane];
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma_tile<bf16>(a[i][q], wf, acc[i][j]);
    }
  };

#pragma unroll
  for (int r = 0; r < kR; ++r) {
    load_w(r, dw[r]);
    load_a(r, da[r]);
  }
  store_w(0, dw[0]);
  __syncthreads();
  // Iteration kt: W of k-tile kt is in LDS buffer kt & 1; its register stage is refilled
  // with k-tile kt + kR; W of k-tile kt + 1 moves to the other buffer.
  const int KTr = KT - KT % kR;
  for (int kt0 = 0; kt0 < KTr; kt0 += kR) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int kt = kt0 + r;
      load_w(kt + kR, dw[r]);
      compute(kt & 1, da[r]);
      load_a(kt + kR, da[r]);
      store_w((kt + 1) & 1, dw[(r + 1) % kR]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < kR - 1; ++r) {
    const int kt = KTr + r;
    if (kt < KT) {
      compute(kt & 1, da[r]);
      store_w((kt + 1) & 1, dw[(r + 1) % kR]);
      __syncthreads();
    }
  }

  {  // 1 / rms of every row of the block
    float ssum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ssum += sq[i];
    for (int part = 8; part < p.ssq_parts; ++part)
      if (my_row < p.M) ssum += p.ssq_in[(long long)part * p.ssq_ld + my_row];
    rstd_s[tid] = 1.0f / sqrtf(ssum / (float)(KT * 32) + p.eps);
  }
  __syncthreads();

  // acc[i][j][e]: row 64 wave + 16 i + 4 (lane / 16) + e, column 16 j + lane % 16.
  const int cols = ntv * 16;
  if constexpr (EPI == EPI_ARGMAX && kQ == 1) {
    // Refine mode: the best three keys of every (row, 128-column part).  The block goes
    // through LDS in two 128-row halves; two threads scan one row (64 columns each, in
    // column order, so among equal values the lower index stays ahead), then merge.  The
    // keys are those of the in-register selection below (NaN values are never picked).
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wave / 2 == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kTallNT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = (wave % 2) * 64 + i * 16 + (lane >> 4) * 4 + e;   // row in the half
              sm.tile[r * kWideLd + j * 16 + (lane & 15)] = acc[i][j][e] * rstd_s[half * kTallM + r];
            }
      }
      __syncthreads();
      const int r = tid >> 1, c0 = (tid & 1) * 64, cend = min(c0 + 64, cols);
      float v1 = -INFINITY, v2 = -INFINITY, v3 = -INFINITY;
      int i1 = -1, i2 = -1, i3 = -1;
      for (int c = c0; c < cend; c += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.tile[r * kWideLd + c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = x[e];
          const bool g1 = v > v1, g2 = v > v2, g3 = v > v3;
          v3 = g2 ? v2 : (g3 ? v : v3);
          i3 = g2 ? i2 : (g3 ? c + e : i3);
          v2 = g1 ? v1 : (g2 ? v : v2);
          i2 = g1 ? i1 : (g2 ? c + e : i2);
          v1 = g1 ? v : v1;
          i1 = g1 ? c + e : i1;
        }
      }
      const int base = cb * kTallN;
      unsigned long long k1 = i1 >= 0 ? argmax_key(v1, base + i1) : 0ull;
      unsigned long long k2 = i2 >= 0 ? argmax_key(v2, base + i2) : 0ull;
      unsigned long long k3 = i3 >= 0 ? argmax_key(v3, base + i3) : 0ull;
      const unsigned long long o1 = __shfl_xor(k1, 1, kWave), o2 = __shfl_xor(k2, 1, kWave),
                               o3 = __shfl_xor(k3, 1, kWave);
      top3_push(k1, k2, k3, o1);
      top3_push(k1, k2, k3, o2);
      top3_push(k1, k2, k3, o3);
      const int m = rb * kWideRows + half * kTallM + r;
      if ((tid & 1) == 0 && m < p.M) {   // row-major [row][part]: one sweep per row later
        const long long ki = (long long)m * p.keys_ld + cb;
        p.keys[ki] = k1;
        p.keys2[ki] = k2;
        p.keys3[ki] = k3;
      }
      __syncthreads();
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = wave * 64 + i * 16 + (lane >> 4) * 4 + e;
        const int m = rb * kWideRows + rl;
        const float rs = rstd_s[rl];
        unsigned long long best = 0, second = 0;
#pragma unroll
        for (int j = 0; j < kTallNT; ++j) {
          const int c = j * 16 + (lane & 15);
          const float v = acc[i][j][e] * rs;
          if (c < cols) {
            top2_push(best, second, argmax_key(v, cb * kTallN + c));
            if (p.logits_out && m < p.M) {
              const long long orow = p.draft_rpr ? draft_out_row(m, p.draft_rpr, p.draft_nb) : m;
              if (orow >= 0) p.logits_out[orow * p.ldo + cb * kTallN + c] = v;
            }
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const unsigned long long o1 = __shfl_xor(best, o, kWave);
          const unsigned long long o2 = __shfl_xor(second, o, kWave);
          top2_merge(best, second, o1, o2);
        }
        if ((lane & 15) == 0 && m < p.M) {
          p.keys[(long long)cb * p.keys_ld + m] = best;
          if (p.keys2) p.keys2[(long long)cb * p.keys_ld + m] = second;
        }
      }
  } else {
    // Two halves of 128 rows through the LDS tile (which reuses the W buffers).
    const int ld = cols + 1;
    const EpiPrefetch<0> pre{};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wave / 2 == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kTallNT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = (wave % 2) * 64 + i * 16 + (lane >> 4) * 4 + e;   // row in the half
              const int col = j * 16 + (lane & 15);
              if (col < cols) sm.tile[r * ld + col] = acc[i][j][e] * rstd_s[half * kTallM + r];
            }
      }
      __syncthreads();
      run_epilogue<bf16, kTallMT, EPI, 0, kTallNT>(p, sm.tile, cols, cb * kTallNT, 2 * rb + half,
                                                  0, cb, pre);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launch
// ------------------------------------------------------------------------------------------
template <typename T, int AK, int MT, int NPW, int EPI, bool NORM>
static hipError_t go(const GemmParams& p, int layers, hipStream_t stream) {
  // The shape must fit the kernel's static resources: workgroup size bound, LDS reduction
  // slots and the epilogue tile; every tile group must be whole.
  const int waves = p.ksub * p.tgpw;
  if (p.ksub < 1 || p.tgpw < 1 || waves > kMaxWaves || waves * NPW * MT > kRedSlots ||
      MT * 16 * (p.tgpw * NPW * 16 + 1) > kTileFloats || p.n_tiles % (p.tgpw * NPW) != 0 ||
      (NPW >= 8 && waves * kWave > 256))
    return hipErrorInvalidValue;
  dim3 grid(p.n_tiles / (p.tgpw * NPW) * p.n_mblocks, 1, layers);
  dim3 block(kWave * p.ksub * p.tgpw);
  gemm_stream<T, AK, MT, NPW, EPI, NORM><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int AK, int MT, int EPI, bool NORM>
static hipError_t by_npw(int npw, const GemmParams& p, int layers, hipStream_t stream) {
  if (npw == 1) return go<T, AK, MT, 1, EPI, NORM>(p, layers, stream);
  if (npw == 2) return go<T, AK, MT, 2, EPI, NORM>(p, layers, stream);
  // 4 n-tiles at 4 m-tiles would not fit the register file with the load ring.
  if constexpr (MT < 4) {
    if (npw == 4) return go<T, AK, MT, 4, EPI, NORM>(p, layers, stream);
  }
  if constexpr (EPI == EPI_ARGMAX && MT == 1) {   // the LM head's wide, single-m-tile case
    if (npw == 8) return go<T, AK, MT, 8, EPI, NORM>(p, layers, stream);
  }
  return hipErrorInvalidValue;
}

// The instantiated (A kind, epilogue, norm) combinations are the ones the drafter uses.
template <typename T, int MT>
static hipError_t launch_mt(int npw, int epi, const GemmParams& p, int layers,
                            hipStream_t stream) {
  const bool norm = p.norm != 0;
  constexpr bool kBf16 = std::is_same<T, bf16>::value;
  switch (p.a_kind) {
    case A_SWZ:   // fp32 models: every activation; bf16 models: the injection's input
      if (epi == EPI_INJECT && !norm) return by_npw<T, A_SWZ, MT, EPI_INJECT, false>(npw, p, layers, stream);
      if constexpr (!kBf16) {
        if (epi == EPI_RESIDUAL && !norm) return by_npw<T, A_SWZ, MT, EPI_RESIDUAL, false>(npw, p, layers, stream);
        if (epi == EPI_QKV && norm) return by_npw<T, A_SWZ, MT, EPI_QKV, true>(npw, p, layers, stream);
        if (epi == EPI_SWIGLU && norm) return by_npw<T, A_SWZ, MT, EPI_SWIGLU, true>(npw, p, layers, stream);
        if (epi == EPI_ARGMAX && norm) return by_npw<T, A_SWZ, MT, EPI_ARGMAX, true>(npw, p, layers, stream);
      }
      break;
    case A_HILO:  // bf16 models: everything the drafter produces except the injection input
      if constexpr (kBf16) {
        if (epi == EPI_RESIDUAL && !norm) return by_npw<T, A_HILO, MT, EPI_RESIDUAL, false>(npw, p, layers, stream);
        if (epi == EPI_QKV && norm) return by_npw<T, A_HILO, MT, EPI_QKV, true>(npw, p, layers, stream);
        if (epi == EPI_SWIGLU && norm) return by_npw<T, A_HILO, MT, EPI_SWIGLU, true>(npw, p, layers, stream);
        if (epi == EPI_ARGMAX && norm) return by_npw<T, A_HILO, MT, EPI_ARGMAX, true>(npw, p, layers, stream);
      }
      break;
    case A_ROW_F32:
      if (epi == EPI_STORE && !norm) return by_npw<T, A_ROW_F32, MT, EPI_STORE, false>(npw, p, layers, stream);
      break;
    case A_ROW_BF16:
      if constexpr (sizeof(T) == 2) {
        if (epi == EPI_STORE && !norm) return by_npw<T, A_ROW_BF16, MT, EPI_STORE, false>(npw, p, layers, stream);
      }
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

// Reduction of a k-split 128-row GEMM: a thread adds the slices' partials of four columns in
// slice order.  EPI_STORE: the sum is the output (fp32 fragment layout); one thread per
// (row, column quad).  EPI_RESIDUAL: the sum is added to x, and x and x * gamma_next (pair
// layout) are written, and the rows' squares are reduced (lanes, then waves, in a fixed
// order) to one partial per 512-column segment for the next norm, so the next
// RMSNorm-folded GEMM reads a few partials per row instead of one per n-tile.
constexpr int kRedSegCols = 512;   // columns per workgroup of the residual reduction
template <int EPI>
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(GemmParams p, int splits) {
  const int quads = p.n_tiles * 4;
  const int kto = p.ldo / 32;
  auto reduce_quad = [&](int m, int cq) -> f32x4 {
    const int col = cq * 4;
    // Four slices' loads in flight at a time, added in slice order.
    constexpr int kU = 4;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += kU) {
      f32x4 t[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        t[u] = s0 + u < splits ? *reinterpret_cast<const f32x4*>(
                                     p.partial + ((long long)(s0 + u) * p.M + m) * p.ldo + col)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (s0 + u < splits) v += t[u];
    }
    f32x4* xp = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + swz_off(m, col, kto, 8));
    const f32x4 xn = EPI == EPI_RESIDUAL ? *xp + v : v;
    *xp = xn;
    return xn;
  };
  if constexpr (EPI == EPI_RESIDUAL) {
    // Workgroup (m-tile, 512-column segment): in the fragment layout the segment of an
    // m-tile is 32 KB contiguous, so thread t takes its 16-byte pieces t + 256 i, all of row
    // t % 16; every load is issued before the first store.  The row's squares over the
    // segment are reduced over the 16 threads of that row (lanes, then waves) to one
    // partial: parts = 512-column segments.
    constexpr int kP = kRedSegCols / 32 * 128 / 256;   // pieces per thread (8)
    __shared__ float red[256 / kWave][16];
    const int mt = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
    const int kt0 = seg * (kRedSegCols / 32), nkt = min(kRedSegCols / 32, kto - kt0);
    const int r = mt * 16 + tid % 16;
    const bool row_ok = r < p.M;
    f32x4 v[kP], xo[kP], g[kP];
    long long xoff[kP];
    int col[kP];
    bool ok[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int pc = tid + 256 * i, ktl = pc / 128, jb = (pc / 64) % 2, ln = pc % 64;
      ok[i] = row_ok && ktl < nkt;
      col[i] = (kt0 + ktl) * 32 + 8 * (ln / 16) + 4 * jb;
      xoff[i] = (((long long)mt * kto + kt0 + ktl) * 2 + jb) * 256 + ln * 4;
      v[i] = xo[i] = g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok[i]) {
        xo[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.out) + xoff[i]);
        if (p.xg_out) g[i] = *reinterpret_cast<const f32x4*>(p.gamma_next + col[i]);
      }
    }
    // The slices' partials are in x's fragment layout (gemm_tall's k-slice epilogue).  The
    // first two slices' loads are all in flight together; further slices follow in order.
    {
      f32x4 s1[kP];
#pragma unroll
      for (int i = 0; i < kP; ++i) {
        s1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ok[i]) {
          v[i] = *reinterpret_cast<const f32x4*>(p.partial + xoff[i]);
          if (splits > 1)
            s1[i] = *reinterpret_cast<const f32x4*>(p.partial + (long long)p.M * p.ldo + xoff[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kP; ++i) {
        v[i] = f32x4{0.f, 0.f, 0.f, 0.f} + v[i];   // the sum starts from 0, as for any slice count
        if (splits > 1) v[i] += s1[i];
      }
    }
    for (int sl = 2; sl < splits; ++sl)
#pragma unroll
      for (int i = 0; i < kP; ++i)
        if (ok[i])
          v[i] += *reinterpret_cast<const f32x4*>(p.partial + (long long)sl * p.M * p.ldo +
                                                 xoff[i]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      if (!ok[i]) continue;
      const f32x4 xn = xo[i] + v[i];
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + xoff[i]) = xn;
      if (p.xg_out) {
        store_hilo4(reinterpret_cast<bf16*>(p.xg_out), hilo_off(r, col[i], kto), xn * g[i]);
        ss += xn[0] * xn[0] + xn[1] * xn[1] + xn[2] * xn[2] + xn[3] * xn[3];
      }
    }
    if (p.xg_out) {
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      if (tid % kWave < 16) red[tid / kWave][tid % 16] = ss;
      __syncthreads();
      if (tid < 16 && r < p.M) {
        float t = 0.f;
        for (int w = 0; w < 256 / kWave; ++w) t += red[w][tid];
        p.ssq_out[(long long)seg * p.ssq_ld + r] = t;
      }
    }
  } else {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx < (long long)p.M * quads) reduce_quad((int)(idx / quads), (int)(idx % quads));
  }
}

// Reduction of a block-wise k-split: kTileSubs workgroups per 128 x 128 output block, each
// taking 32 of its rows, add the slices' partial blocks in slice order (16-byte loads, a
// whole slice's loads in flight at once), apply the rows' RMSNorm scale and run the
// unsplit epilogue on the 32-row tile.
constexpr int kTileSubs = 4, kSubRows = kTallM / kTileSubs;
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void ksplit_tile_reduce_kernel(GemmParams p, int splits) {
  __shared__ float tile[kSubRows * (kTallN + 1)];
  __shared__ float rstd_s[kSubRows];
  __shared__ float ssq_s[256];
  const int tid = threadIdx.x;
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT, nblk = ncb * p.n_mblocks;
  const int blk = blockIdx.x / kTileSubs, sub = blockIdx.x % kTileSubs;
  const int rb = blk / ncb, cb = blk % ncb;
  const int cols = min(kTallNT, p.n_tiles - cb * kTallNT) * 16, ld = cols + 1;
  const int m0 = rb * kTallM + sub * kSubRows;
  const int rows = min(kSubRows, p.M - m0);
  if (rows <= 0) return;
  // The first two slices' loads go out first, all in flight together (further slices follow
  // in order after the norm's sums).
  const int q4 = cols / 4;   // 16-byte chunks per row
  const float* src = p.partial + (long long)blk * (kTallM * kTallN) +
                     (long long)sub * kSubRows * kTallN;
  const long long sstride = (long long)nblk * (kTallM * kTallN);
  constexpr int kPer = kSubRows * kTallN / 4 / 256;   // chunks per thread (full block)
  f32x4 v[kPer], s1[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + j * 256, r = q / q4, c = (q % q4) * 4;
    v[j] = s1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < rows) {
      v[j] = *reinterpret_cast<const f32x4*>(src + r * kTallN + c);
      if (splits > 1) s1[j] = *reinterpret_cast<const f32x4*>(src + sstride + r * kTallN + c);
    }
  }
  if constexpr (NORM) {   // thread t: row t % 32, parts t / 32 + 8 i; then the 8 sums in order
    const int r = tid % kSubRows, m = m0 + r;
    float s = 0.f;
    if (r < rows)
      for (int part = tid / kSubRows; part < p.ssq_parts; part += 256 / kSubRows)
        s += p.ssq_in[(long long)part * p.ssq_ld + m];
    ssq_s[tid] = s;
    __syncthreads();
    if (tid < kSubRows) {
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < 256 / kSubRows; ++g) t += ssq_s[g * kSubRows + tid];
      rstd_s[tid] = 1.0f / sqrtf(t / (float)(p.KT * 32) + p.eps);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f} + v[j];   // the sum starts from 0, as for any slice count
    if (splits > 1) v[j] += s1[j];
  }
  for (int sl = 2; sl < splits; ++sl) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = tid + j * 256, r = q / q4, c = (q % q4) * 4;
      if (r < rows)
        v[j] += *reinterpret_cast<const f32x4*>(src + sl * sstride + r * kTallN + c);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + j * 256, r = q / q4, c = (q % q4) * 4;
    if (r < rows) {
      const float sc = NORM ? rstd_s[r] : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[r * ld + c + e] = v[j][e] * sc;
    }
  }
  __syncthreads();
  const EpiPrefetch<0> pre{};
  run_epilogue<bf16, kSubRows / 16, EPI, 0>(p, tile, cols, cb * kTallNT,
                                             rb * kTileSubs + sub, 0, cb, pre);
}

// ------------------------------------------------------------------------------------------
// The deep-K fusion of bf16 feature rows over 256-row blocks, k split over grid.y: the
// 256-row LM head's scheme (W staged in LDS per k-tile, each wave's 64 rows of A loaded
// straight into registers as fragments -- a bf16 row's 16 bytes at k 8 (l / 16) are lane l's
// fragment -- and every W fragment read from LDS feeding four MFMAs) instead of the 128-row
// kernel's staging of both operands, whose 64 x 64 wave tiles asked for about the LDS peak.
// Each slice writes its fp32 partial to partial[slice][row][col]; ksplit_reduce_kernel
// adds the slices in order.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void gemm_rows256(GemmParams p) {
  __shared__ i32x4 w_s[2][kTallNT][kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT, nrb = (p.M + kWideRows - 1) / kWideRows;
  int cb, rb;   // same XCD-aware order as the 128-row kernel
  if (nrb <= kTallColRows) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    cb = (slot / nrb) * kXcds + xcd;
    rb = slot % nrb;
    if (cb >= ncb) return;
  } else {
    cb = blockIdx.x % ncb;
    rb = blockIdx.x / ncb;
  }
  const int S = max(p.ksplit, 1), sl = blockIdx.y;
  const int kb = (sl * p.KT) / S, KT = ((sl + 1) * p.KT) / S - kb;
  const int ntv = min(kTallNT, p.n_tiles - cb * kTallNT);
  const char* W = p.W + (long long)(p.nt0 + cb * kTallNT) * p.nt_stride * kTileBytes;
  // This wave's 4 m-tiles; rows past M re-read row M - 1 (never stored).
  const bf16* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(rb * kWideRows + wave * 64 + i * 16 + (lane & 15), p.M - 1);
    ap[i] = reinterpret_cast<const bf16*>(p.A) + (long long)row * p.lda + (lane >> 4) * 8;
  }
  constexpr int kR = 2;
  i32x4 da[kR][4], dw[kR][2];
  auto load_a = [&](int kt, i32x4 (&a)[4]) {
    const long long off = (long long)(kb + min(kt, KT - 1)) * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const i32x4*>(ap[i] + off);
  };
  auto load_w = [&](int kt, i32x4 (&w)[2]) {
    const int ktc = kb + min(kt, KT - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256, nt = min(c / 64, ntv - 1), l = c % 64;
      w[i] = load16(W + ((long long)nt * p.nt_stride + (long long)ktc * p.kt_stride) *
                            kTileBytes + l * 16);
    }
  };
  auto store_w = [&](int buf, const i32x4 (&w)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      w_s[buf][c / 64][c % 64] = w[i];
    }
  };
  f32x4 acc[4][kTallNT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kTallNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const i32x4 (&a)[4]) {
#pragma unroll
    for (int j = 0; j < kTallNT; ++j) {
      const i32x4 wf = w_s[buf][j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_tile<bf16>(a[i], wf, acc[i][j]);
    }
  };
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    load_w(r, dw[r]);
    load_a(r, da[r]);
  }
  store_w(0, dw[0]);
  __syncthreads();
  // Iteration kt: W of k-tile kt is in LDS buffer kt & 1; its register stage is refilled
  // with k-tile kt + kR; W of k-tile kt + 1 moves to the other buffer.
  const int KTr = KT - KT % kR;
  for (int kt0 = 0; kt0 < KTr; kt0 += kR) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int kt = kt0 + r;
      load_w(kt + kR, dw[r]);
      compute(kt & 1, da[r]);
      load_a(kt + kR, da[r]);
      store_w((kt + 1) & 1, dw[(r + 1) % kR]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < kR - 1; ++r) {
    const int kt = KTr + r;
    if (kt < KT) {
      compute(kt & 1, da[r]);
      store_w((kt + 1) & 1, dw[(r + 1) % kR]);
      __syncthreads();
    }
  }
  // acc[i][j][e]: row 64 wave + 16 i + 4 (lane / 16) + e, column 16 j + lane % 16.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = rb * kWideRows + wave * 64 + i * 16 + (lane >> 4) * 4 + e;
      if (m >= p.M) continue;
      float* dst = p.partial + ((long long)sl * p.M + m) * p.ldo + cb * kTallN + (lane & 15);
#pragma unroll
      for (int j = 0; j < kTallNT; ++j)
        if (j < ntv) dst[j * 16] = acc[i][j][e];
    }
}

static hipError_t go_rows256(const GemmParams& p, hipStream_t stream) {
  const int splits = std::max(p.ksplit, 1);
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT;
  const int nrb = (p.M + kWideRows - 1) / kWideRows;
  if (!p.partial || p.KT < splits || p.ldo % 16 != 0 || p.lda % 8 != 0 || p.M < 1)
    return hipErrorInvalidValue;
  const int ncb_grid = nrb <= kTallColRows ? (ncb + kXcds - 1) / kXcds * kXcds : ncb;
  gemm_rows256<<<dim3(ncb_grid * nrb, splits, 1), 256, 0, stream>>>(p);
  const long long threads = (long long)p.M * p.n_tiles * 4;
  ksplit_reduce_kernel<EPI_STORE><<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(p, splits);
  return hipGetLastError();
}

template <int AK, int EPI, bool NORM>
static hipError_t go_tall(const GemmParams& p, int layers, hipStream_t stream) {
  const int ncb = (p.n_tiles + kTallNT - 1) / kTallNT;
  const int ncb_grid = p.n_mblocks <= kTallColRows ? (ncb + kXcds - 1) / kXcds * kXcds : ncb;
  const int splits = (kRowSplit<EPI> || kTileSplit<EPI>) ? std::max(p.ksplit, 1) : 1;
  if (splits > 1 && (layers != 1 || !p.partial || p.KT < splits ||
                     (kRowSplit<EPI> && p.ldo % 16 != 0)))
    return hipErrorInvalidValue;
  dim3 grid(ncb_grid * p.n_mblocks, splits, layers);
  gemm_tall<AK, EPI, NORM><<<grid, 256, 0, stream>>>(p);
  if (splits > 1) {
    if constexpr (EPI == EPI_RESIDUAL) {   // a workgroup per (m-tile, 512-column segment)
      const dim3 rg((unsigned)((p.M + 15) / 16), (unsigned)((p.ldo + kRedSegCols - 1) / kRedSegCols));
      ksplit_reduce_kernel<EPI><<<rg, 256, 0, stream>>>(p, splits);
    } else if constexpr (kRowSplit<EPI>) {
      const long long threads = (long long)p.M * p.n_tiles * 4;
      ksplit_reduce_kernel<EPI><<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(p, splits);
    } else if constexpr (kTileSplit<EPI>) {
      ksplit_tile_reduce_kernel<EPI, NORM>
          <<<ncb * p.n_mblocks * kTileSubs, 256, 0, stream>>>(p, splits);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype_bf16, int mt, int npw, int epi, const GemmParams& p,
                       int layers, hipStream_t stream) {
  if (mt == kTallMT) {   // 128-row x 128-column blocks, bf16 weights
    if (!dtype_bf16 || p.n_tiles < 1 || p.M < 1) return hipErrorInvalidValue;
    const bool norm = p.norm != 0;
    if (p.a_kind == A_SWZ && epi == EPI_INJECT && !norm)
      return go_tall<A_SWZ, EPI_INJECT, false>(p, layers, stream);
    if (p.a_kind == A_ROW_BF16 && epi == EPI_STORE && !norm && p.lda % 8 == 0) {
      if (p.rows256) return layers == 1 ? go_rows256(p, stream) : hipErrorInvalidValue;
      return go_tall<A_ROW_BF16, EPI_STORE, false>(p, layers, stream);
    }
    if (p.a_kind != A_HILO) return hipErrorInvalidValue;
    if (epi == EPI_RESIDUAL && !norm) return go_tall<A_HILO, EPI_RESIDUAL, false>(p, layers, stream);
    if (epi == EPI_QKV && norm) return go_tall<A_HILO, EPI_QKV, true>(p, layers, stream);
    // 256-row blocks for the LM head, and for gate|up once they still give two rounds of
    // workgroups (at 512 rows, 384 workgroups of 256 rows left part of the chip idle: gate|up
    // 185 -> 225 us; at 1024 rows they are faster).
    const int ncb_t = (p.n_tiles + kTallNT - 1) / kTallNT;
    const int nrb_w = (p.M + kWideRows - 1) / kWideRows;
    const bool wide = epi == EPI_ARGMAX || (epi == EPI_SWIGLU && ncb_t * nrb_w >= 512);
    if (epi == EPI_SWIGLU && norm && !wide) return go_tall<A_HILO, EPI_SWIGLU, true>(p, layers, stream);
    if ((epi == EPI_SWIGLU || epi == EPI_ARGMAX) && norm) {   // 256-row blocks
      if (layers != 1) return hipErrorInvalidValue;
      const int ncb = ncb_t, nrb = nrb_w;
      const int ncb_grid = nrb <= kTallColRows ? (ncb + kXcds - 1) / kXcds * kXcds : ncb;
      if (epi == EPI_SWIGLU) gemm_tall256<EPI_SWIGLU, 2><<<ncb_grid * nrb, 256, 0, stream>>>(p);
      else if (p.refine) gemm_tall256<EPI_ARGMAX, 1><<<ncb_grid * nrb, 256, 0, stream>>>(p);
      else gemm_tall256<EPI_ARGMAX, 2><<<ncb_grid * nrb, 256, 0, stream>>>(p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (dtype_bf16) {
    if (mt == 1) return launch_mt<bf16, 1>(npw, epi, p, layers, stream);
    if (mt == 2) return launch_mt<bf16, 2>(npw, epi, p, layers, stream);
    if (mt == 4) return launch_mt<bf16, 4>(npw, epi, p, layers, stream);
  } else {
    if (mt == 1) return launch_mt<float, 1>(npw, epi, p, layers, stream);
    if (mt == 2) return launch_mt<float, 2>(npw, epi, p, layers, stream);
    if (mt == 4) return launch_mt<float, 4>(npw, epi, p, layers, stream);
  }
  return hipErrorInvalidValue;
}

// One 256-thread workgroup per row: threads take the parts in strides (8 loads in flight
// each), then a wave-wide and a workgroup-wide maximum (the best two with keys2).
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const unsigned long long* keys,
                                                              const unsigned long long* keys2,
                                                              int parts, int keys_ld, int* ids,
                                                              float* gap, int rows,
                                                              int draft_rpr, int draft_nb) {
  __shared__ unsigned long long red[2][256 / kWave];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid % kWave;
  unsigned long long best = 0, second = 0;
  if (keys2) {
#pragma unroll 4
    for (int q = tid; q < parts; q += 256) {
      const unsigned long long k1 = keys[(long long)q * keys_ld + m];
      const unsigned long long k2 = keys2[(long long)q * keys_ld + m];
      top2_merge(best, second, k1, k2);
    }
  } else {
#pragma unroll 8
    for (int q = tid; q < parts; q += 256) {
      const unsigned long long k = keys[(long long)q * keys_ld + m];
      best = k > best ? k : best;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long o1 = __shfl_xor(best, o, kWave);
    const unsigned long long o2 = __shfl_xor(second, o, kWave);
    top2_merge(best, second, o1, o2);
  }
  if (lane == 0) {
    red[0][tid / kWave] = best;
    red[1][tid / kWave] = second;
  }
  __syncthreads();
  if (tid != 0) return;
  for (int w = 1; w < 256 / kWave; ++w) top2_merge(best, second, red[0][w], red[1][w]);
  const int idx = argmax_key_index(best);
  const float g = argmax_key_value(best) - argmax_key_value(second);
  const long long o = draft_rpr ? draft_out_row(m, draft_rpr, draft_nb) : m;
  if (o >= 0) {
    ids[o] = idx;
    if (gap && keys2) gap[o] = g;
  }
}

// ------------------------------------------------------------------------------------------
// LM-head refinement (see RefineArgs): one 256-thread workgroup per row.
// ------------------------------------------------------------------------------------------
constexpr int kRefineThreads = 256;
constexpr int kRefinePartsPerThread = 8;   // parts <= 2048 (vocab <= 262144 at 128 columns)
constexpr int kRefineMaxCand = 512;        // columns named one by one
constexpr int kRefineMaxOvf = 32;          // whole parts

__global__ __launch_bounds__(kRefineThreads) void argmax_refine_kernel(RefineArgs a) {
  __shared__ float y_s[kRefineMaxHidden];
  __shared__ int cand_s[kRefineMaxCand];
  __shared__ int ovf_s[kRefineMaxOvf];
  __shared__ int n_cand, n_ovf;
  __shared__ unsigned long long red1[kRefineThreads / kWave], red2[kRefineThreads / kWave];
  __shared__ float fred[2][kRefineThreads / kWave];
  __shared__ float sq_s[kRefineThreads];
  constexpr int kWaves = kRefineThreads / kWave;
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const long long o = a.draft_rpr ? draft_out_row(m, a.draft_rpr, a.draft_nb) : m;
  if (o < 0) return;   // uniform over the workgroup
  const int H = a.KT * 32;

  // Best two hi values of the row over all parts (each part's best three are its keys).
  unsigned long long k1[kRefinePartsPerThread], k2[kRefinePartsPerThread];
  unsigned long long k3[kRefinePartsPerThread];
  const long long kb = (long long)m * a.keys_ld;
#pragma unroll
  for (int i = 0; i < kRefinePartsPerThread; ++i) {
    const int q = tid + i * kRefineThreads;
    k1[i] = q < a.parts ? a.keys[kb + q] : 0ull;
    k2[i] = q < a.parts ? a.keys2[kb + q] : 0ull;
    k3[i] = q < a.parts ? a.keys3[kb + q] : 0ull;
  }
  // The row's sum-of-squares partials (thread i holds partial i; at most 256 of them) and
  // its hi / lo pieces, all requested before any is used.
  const float sq_i = tid < a.ssq_parts ? a.ssq[(long long)tid * a.ssq_ld + m] : 0.f;
  const bf16* arow = reinterpret_cast<const bf16*>(a.a);
  constexpr int kYIt = kRefineMaxHidden / (4 * kRefineThreads);
  bf16x4 hv[kYIt], lv[kYIt];
#pragma unroll
  for (int it = 0; it < kYIt; ++it) {
    const int k = 4 * (tid + it * kRefineThreads);
    if (k < H) {
      const long long off = hilo_off(m, k, a.KT);
      hv[it] = *reinterpret_cast<const bf16x4*>(arow + off);
      lv[it] = *reinterpret_cast<const bf16x4*>(arow + off + kHiLoStride);
    }
  }
  unsigned long long best = 0, second = 0;
#pragma unroll
  for (int i = 0; i < kRefinePartsPerThread; ++i) top2_merge(best, second, k1[i], k2[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o1 = __shfl_xor(best, off, kWave);
    const unsigned long long o2 = __shfl_xor(second, off, kWave);
    top2_merge(best, second, o1, o2);
  }
  if (lane == 0) {
    red1[wave] = best;
    red2[wave] = second;
  }
  if (tid == 0) {
    n_cand = 0;
    n_ovf = 0;
  }
  sq_s[tid] = sq_i;
  __syncthreads();
  // 1 / rms as the GEMM forms it (the partials added in order), the exact input row
  // y = (hi + lo) * rstd in LDS, and the norms of lo and of y.
  float ssum = 0.f;
  for (int i = 0; i < a.ssq_parts; ++i) ssum += sq_s[i];
  const float rstd = 1.0f / sqrtf(ssum / (float)H + a.eps);
  float lo2 = 0.f, y2 = 0.f;
#pragma unroll
  for (int it = 0; it < kYIt; ++it) {
    const int k = 4 * (tid + it * kRefineThreads);
    if (k < H) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lj = (float)lv[it][j];
        const float yj = ((float)hv[it][j] + lj) * rstd;
        y_s[k + j] = yj;
        lo2 += lj * lj;
        y2 += yj * yj;
      }
    }
  }
  lo2 = wave_sum(lo2);
  y2 = wave_sum(y2);
  if (lane == 0) {
    fred[0][wave] = lo2;
    fred[1][wave] = y2;
  }
  __syncthreads();
  best = red1[0];
  second = red2[0];
  lo2 = fred[0][0];
  y2 = fred[1][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    top2_merge(best, second, red1[w], red2[w]);
    lo2 += fred[0][w];
    y2 += fred[1][w];
  }
  // Candidate threshold: the second-best hi value minus twice the hi-versus-exact bound,
  // minus the rounding of both fp32 sums (at most H u sum|w y| each, u = 2^-24).
  const float wmax = *a.wmax;
  const float beta = rstd * sqrtf(lo2) * wmax;
  const float ynorm = sqrtf(y2);
  const float v1 = argmax_key_value(best), v2 = argmax_key_value(second);
  const float margin = 4.0f * (float)H * 5.9604645e-8f * wmax * ynorm +
                       1e-6f * (fabsf(v1) + 1.0f);
  const float tau = v2 - 2.0f * beta - margin;
#pragma unroll
  for (int i = 0; i < kRefinePartsPerThread; ++i) {
    const int q = tid + i * kRefineThreads;
    if (q >= a.parts) continue;
    if (k3[i] != 0ull && argmax_key_value(k3[i]) >= tau) {   // more may hide in this part
      const int s = atomicAdd(&n_ovf, 1);
      if (s < kRefineMaxOvf) ovf_s[s] = q;
      continue;
    }
    if (k1[i] != 0ull && argmax_key_value(k1[i]) >= tau) {
      const int s = atomicAdd(&n_cand, 1);
      if (s < kRefineMaxCand) cand_s[s] = argmax_key_index(k1[i]);
    }
    if (k2[i] != 0ull && argmax_key_value(k2[i]) >= tau) {
      const int s = atomicAdd(&n_cand, 1);
      if (s < kRefineMaxCand) cand_s[s] = argmax_key_index(k2[i]);
    }
  }
  __syncthreads();
  const int nc = n_cand, nv = n_ovf;
  const bool all = nc > kRefineMaxCand || nv > kRefineMaxOvf;   // too many: every column
  const int work = all ? a.vocab : nc + nv * a.part_cols;

  // Exact value of each listed column: one wave per column, 8-element chunks of the packed
  // row (tile (v/16, kt), lane (q * 16 + v % 16) holds k = 32 kt + 8 q .. + 8).
  const int nchunks = a.KT * 4;
  best = 0ull;
  second = 0ull;
  for (int it = wave; it < work; it += kWaves) {
    int col;
    if (all) col = it;
    else if (it < nc) col = cand_s[it];
    else col = ovf_s[(it - nc) / a.part_cols] * a.part_cols + (it - nc) % a.part_cols;
    if (col < 0 || col >= a.vocab) continue;   // uniform over the wave
    const char* wt = a.w + (long long)(col >> 4) * a.nt_stride * kTileBytes;
    float sacc = 0.f;
    constexpr int kU = 8;   // chunk loads a lane issues together
    for (int c0 = 0; c0 < nchunks; c0 += kU * kWave) {
      i32x4 wv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * kWave + lane;
        const int kt = c >> 2, q = c & 3;
        wv[u] = c < nchunks ? *reinterpret_cast<const i32x4*>(
                                  wt + (long long)kt * a.kt_stride * kTileBytes +
                                  (q * 16 + (col & 15)) * 16)
                            : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < nchunks) {
          const bf16x8 wb = __builtin_bit_cast(bf16x8, wv[u]);
          const float* yk = y_s + (c >> 2) * 32 + (c & 3) * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j) sacc += (float)wb[j] * yk[j];
        }
      }
    }
    sacc = wave_sum(sacc);
    top2_push(best, second, argmax_key(sacc, col));
  }
  __syncthreads();
  if (lane == 0) {
    red1[wave] = best;
    red2[wave] = second;
  }
  __syncthreads();
  if (tid != 0) return;
  best = red1[0];
  second = red2[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) top2_merge(best, second, red1[w], red2[w]);
  a.ids[o] = argmax_key_index(best);
  if (a.gap) a.gap[o] = argmax_key_value(best) - argmax_key_value(second);
}

hipError_t launch_argmax_refine(const RefineArgs& a, int rows, hipStream_t stream) {
  if (a.KT * 32 > kRefineMaxHidden || a.parts > kRefineThreads * kRefinePartsPerThread ||
      a.part_cols != kTallN || !a.keys2 || !a.keys3 || !a.wmax || a.ssq_parts > kRefineThreads)
    return hipErrorInvalidValue;
  argmax_refine_kernel<<<rows, kRefineThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(const unsigned long long* keys,
                                  const unsigned long long* keys2, int parts, int keys_ld,
                                  int* ids, float* gap, int rows, int draft_rpr, int draft_nb,
                                  hipStream_t stream) {
  argmax_finalize_kernel<<<rows, 256, 0, stream>>>(keys, gap ? keys2 : nullptr, parts, keys_ld,
                                                  ids, gap, rows, draft_rpr, draft_nb);
  return hipGetLastError();
}

}  // namespace dflash
