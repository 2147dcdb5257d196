// Weight-streaming GEMM for the DFlash drafter: out = A . W^T with a fused epilogue.
//
// Weights are bf16 (or fp32 for fp32 models); activations are fp32 in memory and enter a
// bf16 MFMA as a hi + lo pair (see AFrag), except the bf16 target features of the fusion.
// Every drafter GEMM has few rows (16 block slots per request, or the injected context
// rows) and a large weight matrix, so at small batch the kernel's job is to stream the
// packed bf16 weights from HBM at full bandwidth and feed each 16-byte lane chunk straight
// into a 16x16 MFMA step (no LDS staging of W, no reuse to exploit).  Work split:
//   * a workgroup (4 waves) owns `tpw` n-tiles of 16 output columns and one k-split;
//     its waves divide the split's k-tiles (4 / tpw sub-ranges per n-tile) and reduce
//     through LDS in a fixed order;
//   * an epilogue "group" is the set of n-tiles whose outputs must be seen together (a
//     RoPE head, a gate/up pair, an argmax slab).  When a group spans several workgroups
//     (k-splits or wide heads), each writes its partial tile, and the last one to arrive
//     (device-scope counter) sums the partials in split order and runs the epilogue.  The
//     sum order is fixed, so results are bitwise repeatable run to run.
#include "common.h"
#include "gemm.h"

namespace dflash {

constexpr int kThreads = 256;
constexpr int kGroupMax = 8;
constexpr int kUnroll = 8;

template <int MT>
struct GemmSmem {
  f32x4 red[4][MT][kWave];
  float tile[MT * 16][kGroupMax * 16 + 1];
  unsigned flag;
};

template <typename T>
__device__ inline i32x4 load16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// ------------------------------------------------------------------------------------------
// Epilogues: run on the dense fp32 group tile sm.tile[MT*16][group*16].
// ------------------------------------------------------------------------------------------
template <typename T, int MT, int EPI>
__device__ void run_epilogue_impl(const GemmParams& p, GemmSmem<MT>& sm, int group, int mblock,
                             int z) {
  const int g = p.group;
  const int rows = MT * 16;
  const int cols = g * 16;
  const int m0 = mblock * rows;
  const int n0 = group * cols;  // relative to nt0
  const int tid = threadIdx.x;

  if constexpr (EPI == EPI_STORE || EPI == EPI_RESIDUAL) {
    for (int idx = tid; idx < rows * cols; idx += kThreads) {
      const int r = idx / cols, c = idx % cols;
      const int m = m0 + r;
      if (m >= p.M) continue;
      const float v = sm.tile[r][c];
      if constexpr (EPI == EPI_STORE) {
        reinterpret_cast<float*>(p.out)[(long long)m * p.ldo + n0 + c] = v;
      } else {
        float* x = reinterpret_cast<float*>(p.out) + (long long)m * p.ldo + n0 + c;
        *x = *x + v;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = tid; idx < rows * 16; idx += kThreads) {
      const int r = idx / 16, c = idx % 16;
      const int m = m0 + r;
      if (m >= p.M) continue;
      const float gate = sm.tile[r][c];
      const float up = sm.tile[r][16 + c];
      reinterpret_cast<float*>(p.out)[(long long)m * p.ldo + group * 16 + c] =
          silu(gate) * up;
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int d = p.head_dim, half = d / 2;
    const int head = group;
    for (int idx = tid; idx < rows * half; idx += kThreads) {
      const int r = idx / half, i = idx % half;
      const int m = m0 + r;
      if (m >= p.M) continue;
      float x1 = sm.tile[r][i], x2 = sm.tile[r][i + half];
      if constexpr (EPI == EPI_QKV) {
        const int b = m / kBlock, j = m % kBlock;
        const int position = p.ctx_lens[b] + j;
        float* dst;
        if (head < p.n_q + p.n_kv) {
          float cs, sn;
          rope_cos_sin(position, i, d, p.log_theta, &cs, &sn);
          const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
          x1 = y1;
          x2 = y2;
          dst = head < p.n_q ? p.q_out + ((long long)m * p.n_q + head) * d
                             : p.bk_out + ((long long)m * p.n_kv + (head - p.n_q)) * d;
        } else {
          dst = p.bv_out + ((long long)m * p.n_kv + (head - p.n_q - p.n_kv)) * d;
        }
        dst[i] = x1;
        dst[i + half] = x2;
      } else {
        const int seq = p.seq_idx[m];
        const int ps = p.pos[m];
        const int page = p.block_table[(long long)seq * p.max_pages + ps / kPage];
        const int slot = ps % kPage;
        const bool is_k = head < p.n_kv;
        const int h = is_k ? head : head - p.n_kv;
        if (is_k) {
          float cs, sn;
          rope_cos_sin(ps, i, d, p.log_theta, &cs, &sn);
          const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
          x1 = y1;
          x2 = y2;
        }
        T* pool = reinterpret_cast<T*>(is_k ? p.k_pool : p.v_pool);
        T* dst = pool + (long long)z * p.pool_layer_elems +
                 (((long long)page * p.n_kv + h) * kPage + slot) * d;
        dst[i] = Elem<T>::from_f(x1);
        dst[i + half] = Elem<T>::from_f(x2);
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    if (p.logits_out) {
      for (int idx = tid; idx < rows * cols; idx += kThreads) {
        const int r = idx / cols, c = idx % cols;
        const int m = m0 + r;
        if (m < p.M) p.logits_out[(long long)m * p.ldo + n0 + c] = sm.tile[r][c];
      }
    }
    if (tid < rows) {
      const int m = m0 + tid;
      if (m < p.M) {
        float best = sm.tile[tid][0];
        int bi = 0;
        for (int c = 1; c < cols; ++c) {
          const float v = sm.tile[tid][c];
          if (v > best) {
            best = v;
            bi = c;
          }
        }
        atomicMax(&p.keys[(long long)m * 16], argmax_key(best, n0 + bi));
      }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) sm.flag = (arrive_counter(p.done_counter) == (unsigned)(p.total_wgs - 1));
    __syncthreads();
    if (sm.flag) {
      __threadfence();
      for (int m = tid; m < p.M; m += kThreads) {
        unsigned long long* kp = &p.keys[(long long)m * 16];
        const unsigned long long k =
            __hip_atomic_load(kp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.ids_out[m] = argmax_key_index(k);
        __hip_atomic_store(kp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (tid == 0)
        __hip_atomic_store(p.done_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Main kernel
// ------------------------------------------------------------------------------------------
template <typename T, typename AT, int MT, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_stream(GemmParams p) {
  __shared__ GemmSmem<MT> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int ksub = 4 / p.tpw;
  const int wgn = blockIdx.x / p.splits;
  const int split = blockIdx.x % p.splits;
  const int mblock = blockIdx.y;
  const int z = blockIdx.z;
  const int tile_in_wg = wave / ksub;
  const int ks = wave % ksub;
  const int nt_rel = wgn * p.tpw + tile_in_wg;

  // k-tile range of this wave
  const int k0 = split * p.kts;
  const int k1 = min(k0 + p.kts, p.KT);
  const int kw = (k1 - k0 + ksub - 1) / ksub;
  const int kb = min(k0 + ks * kw, k1);
  const int ke = min(kb + kw, k1);

  const char* wp = p.W + (long long)z * p.w_zstride +
                   (long long)(p.nt0 + nt_rel) * p.KT * kTileBytes + lane * 16;
  const AT* A = reinterpret_cast<const AT*>(p.A);
  const int m_base = mblock * MT * 16;
  const AT* arow[MT];
  bool aval[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = m_base + mt * 16 + (lane & 15);
    aval[mt] = r < p.M;
    arow[mt] = A + (long long)(aval[mt] ? r : 0) * p.lda + (lane >> 4) * Elem<T>::kPerLane;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const i32x4 zero = {0, 0, 0, 0};
  // The injection GEMM writes the bf16 KV cache: carry its input at full fp32 precision so
  // the stored values round from as close to the exact product as fp32 accumulation allows.
  typedef AFrag<T, AT, EPI == EPI_INJECT ? 3 : 2> Frag;
  for (int kt = kb; kt < ke; kt += kUnroll) {
    i32x4 b[kUnroll];
    Frag a[kUnroll][MT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      b[u] = (kt + u < ke) ? load16<T>(wp + (long long)(kt + u) * kTileBytes) : zero;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[u][mt].load(arow[mt] + (long long)(kt + u) * Elem<T>::kTile, kt + u < ke && aval[mt]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < Frag::kTerms; ++t)
          acc[mt] = mfma_tile<T>(a[u][mt].part[t], b[u], acc[mt]);
  }

  // Reduce the k sub-ranges of one n-tile inside the workgroup, in wave order.
  if (ksub > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sm.red[wave][mt][lane] = acc[mt];
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 s = sm.red[wave][mt][lane];
        for (int q = 1; q < ksub; ++q) s += sm.red[wave + q][mt][lane];
        acc[mt] = s;
      }
    }
  }

  const int g = p.group;
  const int n_groups = p.n_tiles / g;
  const int cols_per_group = g / p.tpw;  // workgroup columns per group
  const int group = (wgn * p.tpw) / g;
  const int wgcol = wgn % cols_per_group;
  const int targets = cols_per_group * p.splits;

  if (targets == 1) {
    if (ks == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sm.tile[mt * 16 + (lane >> 4) * 4 + j][tile_in_wg * 16 + (lane & 15)] = acc[mt][j];
    }
    __syncthreads();
  } else {
    const long long gm = ((long long)z * n_groups + group) * p.n_mblocks + mblock;
    const int slot = split * cols_per_group + wgcol;
    f32x4* part = reinterpret_cast<f32x4*>(p.partials);
    if (ks == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        part[(((gm * targets + slot) * p.tpw + tile_in_wg) * MT + mt) * kWave + lane] = acc[mt];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
      sm.flag = (arrive_counter(&p.counters[gm]) == (unsigned)(targets - 1));
    __syncthreads();
    if (!sm.flag) return;
    __threadfence();
    for (int idx = threadIdx.x; idx < g * MT * kWave; idx += kThreads) {
      const int t = idx / (MT * kWave);
      const int mt = (idx / kWave) % MT;
      const int ln = idx % kWave;
      const int col = t / p.tpw, tiw = t % p.tpw;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < p.splits; ++sp) {
        const int sl = sp * cols_per_group + col;
        s += part[(((gm * targets + sl) * p.tpw + tiw) * MT + mt) * kWave + ln];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.tile[mt * 16 + (ln >> 4) * 4 + j][t * 16 + (ln & 15)] = s[j];
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&p.counters[gm], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  run_epilogue_impl<T, MT, EPI>(p, sm, group, mblock, z);
}

template <typename T, typename AT, int MT>
static hipError_t launch_mt(int epi, const GemmParams& p, int layers, hipStream_t stream) {
  dim3 grid((p.n_tiles / p.tpw) * p.splits, p.n_mblocks, layers);
  dim3 block(kThreads);
  if constexpr (sizeof(AT) == 2) {
    // bf16 activations only occur as the target features entering the fusion GEMM.
    if (epi != EPI_STORE) return hipErrorInvalidValue;
    gemm_stream<T, AT, MT, EPI_STORE><<<grid, block, 0, stream>>>(p);
  } else {
    switch (epi) {
      case EPI_STORE: gemm_stream<T, AT, MT, EPI_STORE><<<grid, block, 0, stream>>>(p); break;
      case EPI_RESIDUAL: gemm_stream<T, AT, MT, EPI_RESIDUAL><<<grid, block, 0, stream>>>(p); break;
      case EPI_SWIGLU: gemm_stream<T, AT, MT, EPI_SWIGLU><<<grid, block, 0, stream>>>(p); break;
      case EPI_QKV: gemm_stream<T, AT, MT, EPI_QKV><<<grid, block, 0, stream>>>(p); break;
      case EPI_INJECT: gemm_stream<T, AT, MT, EPI_INJECT><<<grid, block, 0, stream>>>(p); break;
      case EPI_ARGMAX: gemm_stream<T, AT, MT, EPI_ARGMAX><<<grid, block, 0, stream>>>(p); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename T, typename AT>
static hipError_t launch_a(int mt, int epi, const GemmParams& p, int layers, hipStream_t stream) {
  if (mt == 1) return launch_mt<T, AT, 1>(epi, p, layers, stream);
  if (mt == 2) return launch_mt<T, AT, 2>(epi, p, layers, stream);
  if (mt == 4) return launch_mt<T, AT, 4>(epi, p, layers, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype_bf16, int a_bf16, int mt, int epi, const GemmParams& p,
                       int layers, hipStream_t stream) {
  if (dtype_bf16)
    return a_bf16 ? launch_a<bf16, bf16>(mt, epi, p, layers, stream)
                  : launch_a<bf16, float>(mt, epi, p, layers, stream);
  if (a_bf16) return hipErrorInvalidValue;
  return launch_a<float, float>(mt, epi, p, layers, stream);
}

}  // namespace dflash
