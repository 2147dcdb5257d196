// Block attention of the DFlash draft pass: the 16 block queries of every head of one KV
// group attend, without a mask, to the request's injected context (paged KV cache) and to
// the 16 block keys.
//
// Grid (nc + 1, n_kv, batch).  Workgroup c < nc handles context keys
// [c*chunk, min((c+1)*chunk, T_b)); workgroup nc handles the 16 block keys.  All query
// heads of the KV group are packed as rows r = j*G + hh (G = n_q / n_kv), so one pass over a
// K/V page serves G heads.  K/V pages are staged through LDS 32 keys at a time and an online
// softmax keeps (max, sum, unnormalized output) per row.  Every workgroup writes its
// partial; the last one to arrive merges them in chunk order (log-sum-exp rescaling), so the
// result is independent of scheduling.
#include "attention.h"
#include "common.h"

namespace dflash {

constexpr int kKC = 32;  // keys per LDS stage

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void block_attention_kernel(AttnArgs a) {
  constexpr int G = R / kBlock;
  constexpr int OPH = 256 / D;   // row phases of the output layout
  constexpr int NRO = R / OPH;   // output rows per thread
  constexpr int SPH = 256 / kKC; // row phases of the score layout
  constexpr int NRS = R / SPH;   // score rows per thread
  __shared__ float q_s[R][D + 1];
  __shared__ float k_s[kKC][D + 1];
  __shared__ float v_s[kKC][D];
  __shared__ float p_s[R][kKC + 1];
  __shared__ float m_s[R], l_s[R], sc_s[R];
  __shared__ unsigned flag;

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int nq = a.n_q, nkv = a.n_kv;
  const int T_b = a.ctx_lens[b];
  const bool is_block = c == a.nc;
  int kbeg, kend;
  if (is_block) {
    kbeg = 0;
    kend = kBlock;
  } else {
    kbeg = min((long long)c * a.chunk, (long long)T_b);
    kend = min(kbeg + a.chunk, T_b);
  }

  for (int idx = tid; idx < R * D; idx += 256) {
    const int r = idx / D, i = idx % D;
    const int j = r / G, hh = r % G;
    q_s[r][i] = a.q[((long long)(b * kBlock + j) * nq + g * G + hh) * D + i] * a.scale;
  }
  if (tid < R) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float o[NRO];
#pragma unroll
  for (int n = 0; n < NRO; ++n) o[n] = 0.f;
  __syncthreads();

  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  for (int k0 = kbeg; k0 < kend; k0 += kKC) {
    const int nk = min(kKC, kend - k0);
    for (int idx = tid; idx < kKC * D; idx += 256) {
      const int kk = idx / D, i = idx % D;
      float kv = 0.f, vv = 0.f;
      if (kk < nk) {
        const int t = k0 + kk;
        if (is_block) {
          const long long off = ((long long)(b * kBlock + t) * nkv + g) * D + i;
          kv = a.bk[off];
          vv = a.bv[off];
        } else {
          const int page = a.block_table[(long long)b * a.max_pages + t / kPage];
          const long long off = (((long long)page * nkv + g) * kPage + t % kPage) * D + i;
          kv = Elem<T>::to_f(kpool[off]);
          vv = Elem<T>::to_f(vpool[off]);
        }
      }
      k_s[kk][i] = kv;
      v_s[kk][i] = vv;
    }
    __syncthreads();
    {
      const int cc = tid % kKC, r0 = tid / kKC;
      float s[NRS];
#pragma unroll
      for (int n = 0; n < NRS; ++n) s[n] = 0.f;
      for (int i = 0; i < D; ++i) {
        const float kv = k_s[cc][i];
#pragma unroll
        for (int n = 0; n < NRS; ++n) s[n] += q_s[r0 + n * SPH][i] * kv;
      }
#pragma unroll
      for (int n = 0; n < NRS; ++n) p_s[r0 + n * SPH][cc] = cc < nk ? s[n] : -INFINITY;
    }
    __syncthreads();
    if (tid < R) {
      const float mold = m_s[tid];
      float mx = mold;
      for (int cc = 0; cc < nk; ++cc) mx = fmaxf(mx, p_s[tid][cc]);
      const float sc = expf(mold - mx);
      float l = l_s[tid] * sc;
      for (int cc = 0; cc < kKC; ++cc) {
        const float pe = cc < nk ? expf(p_s[tid][cc] - mx) : 0.f;
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
        for (int cc = 0; cc < kKC; ++cc) acc += p_s[r][cc] * v_s[cc][i];
        o[n] = acc;
      }
    }
    __syncthreads();
  }

  // Partial of this chunk.
  const long long slot = ((long long)b * nkv + g) * (a.nc + 1);
  {
    const int i = tid % D, r0 = tid / D;
#pragma unroll
    for (int n = 0; n < NRO; ++n) {
      const int r = r0 + n * OPH;
      a.part_o[((slot + c) * R + r) * D + i] = o[n];
    }
    if (tid < R) {
      a.part_ml[((slot + c) * R + tid) * 2 + 0] = m_s[tid];
      a.part_ml[((slot + c) * R + tid) * 2 + 1] = l_s[tid];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0)
    flag = arrive_counter(&a.counters[(long long)b * nkv + g]) == (unsigned)a.nc;
  __syncthreads();
  if (!flag) return;
  __threadfence();

  // Merge the nc + 1 partials in chunk order.
  {
    const int i = tid % D, r0 = tid / D;
    float* out = a.out;
#pragma unroll
    for (int n = 0; n < NRO; ++n) {
      const int r = r0 + n * OPH;
      float M = -INFINITY;
      for (int cc = 0; cc <= a.nc; ++cc) {
        const float l = a.part_ml[((slot + cc) * R + r) * 2 + 1];
        if (l > 0.f) M = fmaxf(M, a.part_ml[((slot + cc) * R + r) * 2 + 0]);
      }
      float L = 0.f, acc = 0.f;
      for (int cc = 0; cc <= a.nc; ++cc) {
        const float l = a.part_ml[((slot + cc) * R + r) * 2 + 1];
        if (l > 0.f) {
          const float w = expf(a.part_ml[((slot + cc) * R + r) * 2 + 0] - M);
          L += l * w;
          acc += a.part_o[((slot + cc) * R + r) * D + i] * w;
        }
      }
      const int j = r / G, hh = r % G;
      out[(long long)(b * kBlock + j) * (nq * D) + (g * G + hh) * D + i] = acc / L;
    }
  }
  if (tid == 0)
    __hip_atomic_store(&a.counters[(long long)b * nkv + g], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
static hipError_t launch_t(const AttnArgs& a, int batch, hipStream_t stream) {
  dim3 grid(a.nc + 1, a.n_kv, batch);
  const int G = a.n_q / a.n_kv;
  const int R = G * kBlock;
  if (a.head_dim == 128) {
    if (R == 32) block_attention_kernel<T, 128, 32><<<grid, 256, 0, stream>>>(a);
    else if (R == 64) block_attention_kernel<T, 128, 64><<<grid, 256, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else if (a.head_dim == 64) {
    if (R == 32) block_attention_kernel<T, 64, 32><<<grid, 256, 0, stream>>>(a);
    else if (R == 64) block_attention_kernel<T, 64, 64><<<grid, 256, 0, stream>>>(a);
    else if (R == 128) block_attention_kernel<T, 64, 128><<<grid, 256, 0, stream>>>(a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_attention(int bf16_dtype, const AttnArgs& a, int batch,
                                  hipStream_t stream) {
  return bf16_dtype ? launch_t<bf16>(a, batch, stream) : launch_t<float>(a, batch, stream);
}

bool block_attention_supported(int head_dim, int group) {
  const int R = group * kBlock;
  if (head_dim == 128) return R == 32 || R == 64;
  if (head_dim == 64) return R == 32 || R == 64 || R == 128;
  return false;
}

}  // namespace dflash
