// Small kernels of the DFlash step: weight packing, block embedding, RMSNorm,
// greedy verification and workspace clearing.
#include <type_traits>

#include "common.h"
#include "small.h"

namespace dflash {

// ------------------------------------------------------------------------------------------
// Weight packing into the MFMA tile layout (see gemm.h).  One thread writes one 16-byte lane
// chunk.  Destination n-tile `dt`, tile row `rho` takes its source row as follows:
//   PACK_CONCAT:  segments stacked along N; the first `rope_segs` segments are RoPE heads of
//                 width d whose tile t holds dims 8t + rho/2 (+ d/2 for odd rho), so each
//                 rotation pair lands in two adjacent output columns.
//   PACK_GATE_UP: tile j holds rows 8j..8j+7 of segment 0 (gate) then of segment 1 (up).
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ void pack_kernel(PackArgs a) {
  const long long chunk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)a.n_tiles_total * a.KT * kWave;
  if (chunk >= total) return;
  const int lane = (int)(chunk % kWave);
  const long long tile = chunk / kWave;
  const int kt = (int)(tile % a.KT);
  const int dt = (int)(tile / a.KT);
  const int rho = lane & 15;
  int seg, row;
  if (a.mode == PACK_GATE_UP) {
    seg = rho < 8 ? 0 : 1;
    row = dt * 8 + (rho & 7);
  } else {
    seg = 0;
    int st = dt;
    while (seg + 1 < a.n_segs && st >= a.seg_tiles[seg]) {
      st -= a.seg_tiles[seg];
      ++seg;
    }
    if (seg < a.rope_segs) {
      const int tph = a.head_dim / 16;
      const int head = st / tph, t = st % tph;
      row = head * a.head_dim + 8 * t + (rho >> 1) + (rho & 1) * (a.head_dim / 2);
    } else {
      row = st * 16 + rho;
    }
  }
  const long long col = (long long)kt * Elem<T>::kTile + (lane >> 4) * Elem<T>::kPerLane;
  const T* src = reinterpret_cast<const T*>(a.src[seg]) + (long long)row * a.K + col;
  i32x4 v = *reinterpret_cast<const i32x4*>(src);
  reinterpret_cast<i32x4*>(a.dst)[chunk] = v;
}

hipError_t launch_pack(int bf16_dtype, const PackArgs& a, hipStream_t stream) {
  const long long total = (long long)a.n_tiles_total * a.KT * kWave;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  if (bf16_dtype)
    pack_kernel<bf16><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(a);
  else
    pack_kernel<float><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(a);
  return hipGetLastError();
}

// Norm gains widened to fp32.
template <typename T>
__global__ void widen_kernel(const T* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = Elem<T>::to_f(src[i]);
}

hipError_t launch_widen(int bf16_dtype, const void* src, float* dst, int n, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  if (bf16_dtype)
    widen_kernel<bf16><<<blocks, threads, 0, stream>>>(reinterpret_cast<const bf16*>(src), dst, n);
  else
    widen_kernel<float><<<blocks, threads, 0, stream>>>(reinterpret_cast<const float*>(src), dst,
                                                        n);
  return hipGetLastError();
}

// Sum over a 256-thread workgroup in a fixed order.
__device__ inline float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Euclidean norm of every row of a row-major [rows][cols] matrix: one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void row_norms_kernel(const T* __restrict__ w, int rows,
                                                        int cols, float* __restrict__ norms) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const T* r = w + (long long)row * cols;
  float ss = 0.f;
  for (int c = lane; c < cols; c += kWave) {
    const float v = Elem<T>::to_f(r[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if (lane == 0) norms[row] = sqrtf(ss);
}

// The largest of n values, by one workgroup.
__global__ __launch_bounds__(256) void max_kernel(const float* __restrict__ v, int n,
                                                  float* __restrict__ out) {
  __shared__ float red[256];
  float mx = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) mx = fmaxf(mx, v[i]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

hipError_t launch_row_norm_max(int bf16_dtype, const void* w, int rows, int cols, float* norms,
                               float* out_max, hipStream_t stream) {
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (bf16_dtype)
    row_norms_kernel<bf16><<<blocks, 256, 0, stream>>>(reinterpret_cast<const bf16*>(w), rows,
                                                       cols, norms);
  else
    row_norms_kernel<float><<<blocks, 256, 0, stream>>>(reinterpret_cast<const float*>(w), rows,
                                                        cols, norms);
  max_kernel<<<1, 256, 0, stream>>>(norms, rows, out_max);
  return hipGetLastError();
}

// Block embedding: row b*rpr + j of x is the embedding of the anchor (j = 0) or of the mask
// token (j >= 1; the padding rows of an 8-token block too), widened to fp32 and written in
// the fragment layout (4 columns per store), together with x * gamma of the first RMSNorm
// (pair fragment layout for bf16 models) and the row's sum of squares.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / a.rpr, j = m % a.rpr;
  const int tok = j == 0 ? a.anchor_ids[b] : a.mask_id;
  const T* e = reinterpret_cast<const T*>(a.embed) + (long long)tok * a.hidden;
  constexpr int kPer = Elem<T>::kPerLane;
  const int KT = a.hidden / (4 * kPer);
  float ss = 0.f;
  // Four chunks of 4 values per thread per trip, all loaded before the first store.
  constexpr int kU = 4;
  for (int i0 = 4 * threadIdx.x; i0 < a.hidden; i0 += 4 * blockDim.x * kU) {
    f32x4 v[kU], g[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * 4 * blockDim.x;
      v[u] = g[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < a.hidden) {
        v[u] = f32x4{Elem<T>::to_f(e[i]), Elem<T>::to_f(e[i + 1]), Elem<T>::to_f(e[i + 2]),
                     Elem<T>::to_f(e[i + 3])};
        g[u] = *reinterpret_cast<const f32x4*>(a.gamma + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * 4 * blockDim.x;
      if (i >= a.hidden) continue;
      const long long off = swz_off(m, i, KT, kPer);
      *reinterpret_cast<f32x4*>(a.x + off) = v[u];
      if constexpr (std::is_same<T, bf16>::value)
        store_hilo4(reinterpret_cast<bf16*>(a.xg), hilo_off(m, i, a.hidden / 32), v[u] * g[u]);
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.xg) + off) = v[u] * g[u];
      ss += v[u][0] * v[u][0] + v[u][1] * v[u][1] + v[u][2] * v[u][2] + v[u][3] * v[u][3];
    }
  }
  ss = block_sum256(ss, red);
  if (threadIdx.x == 0) a.ssq[m] = ss;
}

hipError_t launch_embed(int bf16_dtype, const EmbedArgs& a, int rows, hipStream_t stream) {
  if (bf16_dtype)
    embed_kernel<bf16><<<rows, 256, 0, stream>>>(a);
  else
    embed_kernel<float><<<rows, 256, 0, stream>>>(a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void rows_to_fragments_kernel(const float* __restrict__ src,
                                                                int cols, int hilo,
                                                                const float* __restrict__ gamma,
                                                                void* __restrict__ dst,
                                                                float* __restrict__ ssq) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  float ss = 0.f;
  for (int c = 4 * threadIdx.x; c < cols; c += 4 * blockDim.x) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (long long)r * cols + c);
    const f32x4 g = *reinterpret_cast<const f32x4*>(gamma + c);
    if (hilo)
      store_hilo4(reinterpret_cast<bf16*>(dst), hilo_off(r, c, cols / 32), v * g);
    else
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + swz_off(r, c, cols / 16, 4)) =
          v * g;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum256(ss, red);
  if (threadIdx.x == 0) ssq[r] = ss;
}

// Input rows of the input-fusion prefill: x (fp32 fragment layout, rows < n_valid written by
// the fusion GEMM) gives x * gamma and the row's sum of squares, as the embedding kernel does
// for a draft block; rows n_valid .. rows-1 (the last 16-row group's padding) become zero in
// x, x * gamma and the sums.
template <typename T>
__global__ __launch_bounds__(256) void prefill_rows_kernel(float* x, int hidden, int n_valid,
                                                           const float* gamma, void* xg,
                                                           float* ssq) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  constexpr int kPer = Elem<T>::kPerLane;
  const int KT = hidden / (4 * kPer);
  const bool pad = m >= n_valid;
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < hidden; i += 4 * blockDim.x) {
    const long long off = swz_off(m, i, KT, kPer);
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (pad) *reinterpret_cast<f32x4*>(x + off) = v;
    else v = *reinterpret_cast<const f32x4*>(x + off);
    const f32x4 g = *reinterpret_cast<const f32x4*>(gamma + i);
    if constexpr (std::is_same<T, bf16>::value)
      store_hilo4(reinterpret_cast<bf16*>(xg), hilo_off(m, i, hidden / 32), v * g);
    else
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(xg) + off) = v * g;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum256(ss, red);
  if (threadIdx.x == 0) ssq[m] = ss;
}

hipError_t launch_prefill_rows(int bf16_dtype, float* x, int rows, int n_valid, int hidden,
                               const float* gamma, void* xg, float* ssq, hipStream_t stream) {
  if (bf16_dtype)
    prefill_rows_kernel<bf16><<<rows, 256, 0, stream>>>(x, hidden, n_valid, gamma, xg, ssq);
  else
    prefill_rows_kernel<float><<<rows, 256, 0, stream>>>(x, hidden, n_valid, gamma, xg, ssq);
  return hipGetLastError();
}

// Context length seen by each 16-row group of an input-fusion prefill chunk: group g of a
// chunk starting r0 rows into the prefill of request `seq` sees ctx_lens[seq] + r0 + 16 g
// cached positions.
__global__ void prefill_groups_kernel(const int* __restrict__ ctx_lens, int seq, int r0,
                                      int groups, int* __restrict__ group_ctx) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g < groups) group_ctx[g] = ctx_lens[seq] + r0 + kQRows * g;
}

hipError_t launch_prefill_groups(const int* ctx_lens, int seq, int r0, int groups,
                                 int* group_ctx, hipStream_t stream) {
  prefill_groups_kernel<<<(groups + 255) / 256, 256, 0, stream>>>(ctx_lens, seq, r0, groups,
                                                                  group_ctx);
  return hipGetLastError();
}

hipError_t launch_rows_to_fragments(const float* src, int rows, int cols, int hilo,
                                    const float* gamma, void* dst, float* ssq,
                                    hipStream_t stream) {
  rows_to_fragments_kernel<<<rows, 256, 0, stream>>>(src, cols, hilo, gamma, dst, ssq);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Greedy verification, one wave per request, for a block of nb tokens (nd = nb - 1 drafts).
// Lane i < nd compares d_{i+1} with t_i; the ballot of mismatches gives m = index of the
// lowest mismatching lane (nd if none), with no data-dependent branch.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void verify_greedy_kernel(const int* __restrict__ draft,
                                                           const int* __restrict__ target,
                                                           int nb, int* __restrict__ accept,
                                                           int* __restrict__ bonus,
                                                           int* __restrict__ emitted) {
  const int b = blockIdx.x;
  const int l = threadIdx.x;
  const int nd = nb - 1;
  const int d = l < nd ? draft[(long long)b * nd + l] : 0;
  const int t = l < nb ? target[(long long)b * nb + l] : 0;
  const unsigned long long miss = __ballot(l < nd && d != t) | (1ull << nd);
  const int m = __ffsll((long long)miss) - 1;  // lowest set bit
  if (l == 0) {
    accept[b] = m + 1;
    bonus[b] = target[(long long)b * nb + m];
  }
  if (emitted && l < nb) {
    const int tm = __shfl(t, m, kWave);
    emitted[(long long)b * nb + l] = l < m ? d : (l == m ? tm : -1);
  }
}

hipError_t launch_verify_greedy(const int* draft, const int* target, int batch, int nb,
                                int* accept, int* bonus, int* emitted, hipStream_t stream) {
  verify_greedy_kernel<<<batch, 64, 0, stream>>>(draft, target, nb, accept, bonus, emitted);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Closed-loop bookkeeping after a verify: the block's nb positions become the injection
// rows of the next fuse-inject call, then the context grows by the accepted length and the
// bonus token becomes the next anchor.  One wave per request; every lane reads T_b before
// lane 0 rewrites it (the store depends on the loaded value).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void advance_kernel(const int* __restrict__ accept,
                                                     const int* __restrict__ bonus, int nb,
                                                     int max_ctx, int* ctx_lens,
                                                     int* __restrict__ anchors,
                                                     int* __restrict__ inj_seq,
                                                     int* __restrict__ inj_pos) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int T = ctx_lens[b];
  if (l < nb) {
    inj_seq[(long long)b * nb + l] = b;
    inj_pos[(long long)b * nb + l] = min(max(T + l, 0), max_ctx - 1);
  }
  if (l == 0) {
    ctx_lens[b] = T + accept[b];
    anchors[b] = bonus[b];
  }
}

hipError_t launch_advance(const int* accept, const int* bonus, int batch, int nb, int max_ctx,
                          int* ctx_lens, int* anchors, int* inj_seq, int* inj_pos,
                          hipStream_t stream) {
  advance_kernel<<<batch, 64, 0, stream>>>(accept, bonus, nb, max_ctx, ctx_lens, anchors,
                                           inj_seq, inj_pos);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Zero fill (used for the workspace synchronization area; a kernel, not a memset node, so
// it is safe inside captured graphs).
// ------------------------------------------------------------------------------------------
__global__ void fill_zero_kernel(i32x4* p, long long n16) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = i32x4{0, 0, 0, 0};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const long long n16 = (long long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int threads = 256;
  fill_zero_kernel<<<(unsigned)((n16 + threads - 1) / threads), threads, 0, stream>>>(
      reinterpret_cast<i32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace dflash
