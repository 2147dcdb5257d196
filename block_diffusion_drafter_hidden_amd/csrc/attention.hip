// Block attention of the DFlash draft pass: the 16 block queries of every head of one KV
// group attend, without a mask, to the request's injected context (paged KV cache) and to
// the 16 block keys.
//
// Pass 1 (partials), grid (nc + 1, n_kv, batch): workgroup c < nc covers context keys
// [c*chunk, min((c+1)*chunk, T_b)); workgroup nc covers the 16 block keys.  All G query
// heads of the KV group are handled together, one 16-row tile per head (rows = block
// slots), so one pass over a K/V page serves G heads.  Each workgroup keeps an online
// softmax (running max m, sum l, unnormalized output o) and writes (m, l, o).
// Pass 2 (merge), grid (n_q, batch): rescales the nc + 1 partials of each head to a common
// maximum and divides by the total sum, in chunk order, so results do not depend on
// scheduling.
//
// bf16 models run QK^T and PV on 16x16x32 bf16 MFMA: cache K/V are exact bf16 operands,
// fp32 queries, probabilities and block keys/values enter as hi + lo bf16 pairs (products
// of the two lo pieces, ~2^-32 relative, are dropped).  K is staged in LDS row-major, V
// transposed, so every MFMA B fragment is one 16-byte LDS read.  fp32 models use a VALU
// version of pass 1 with the same partial layout.
#include "attention.h"
#include "common.h"

namespace dflash {

constexpr int kKeys = 32;       // keys per step (one MFMA k range of PV)
constexpr int kThreads = 256;   // 4 waves

// ------------------------------------------------------------------------------------------
// bf16: MFMA partial kernel
// ------------------------------------------------------------------------------------------
template <int D, int G>
struct AttnSmem {
  static constexpr int kLd = D + 8;          // K row stride (bf16), padded against conflicts
  static constexpr int vLd = kKeys + 8;      // V^T row stride (bf16)
  bf16 k[2][kKeys][kLd];                     // [piece][key][dim]
  bf16 vt[2][D][vLd];                        // [piece][dim][key]
  float p[4][16][kKeys + 1];                 // per-wave probability tile (row, key)
};

__device__ inline void split2(float v, bf16& hi, bf16& lo) {
  hi = (bf16)v;
  lo = (bf16)(v - (float)hi);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void attn_partial_bf16(AttnArgs a) {
  __shared__ AttnSmem<D, G> sm;
  constexpr int KS = D / 32;            // k-steps of QK^T
  constexpr int DT = D / 16;            // dim tiles of PV
  constexpr int RT = (G + 3) / 4;       // row tiles (heads) per wave
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nq = a.n_q, nkv = a.n_kv;
  const int T_b = a.ctx_lens[b];
  const bool is_block = c == a.nc;
  int kbeg, kend;
  if (is_block) {
    kbeg = 0;
    kend = kBlock;
  } else {
    kbeg = (int)min((long long)c * a.chunk, (long long)T_b);
    kend = min(kbeg + a.chunk, T_b);
  }
  const int npieces = is_block ? 2 : 1;

  // Query fragments (A operand of QK^T): lane l holds row l%16 (block slot), dims
  // 32*ks + 8*(l/16) .. +8, split into hi/lo; scaled by 1/sqrt(d).
  i32x4 qf[RT][KS][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int hh = wave + 4 * rt;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 h, l;
      if (hh < G) {
        const float* src = a.q + ((long long)(b * kBlock + (lane & 15)) * nq + g * G + hh) * D +
                           ks * 32 + (lane >> 4) * 8;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
        const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          bf16 hb, lb;
          split2(f[i] * a.scale, hb, lb);
          h[i] = hb;
          l[i] = lb;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = l[i] = (bf16)0.f;
      }
      qf[rt][ks][0] = __builtin_bit_cast(i32x4, h);
      qf[rt][ks][1] = __builtin_bit_cast(i32x4, l);
    }
  }

  f32x4 o[RT][DT];
  float mrow[RT][4], lrow[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mrow[rt][i] = -INFINITY;
      lrow[rt][i] = 0.f;
    }
  }

  const bf16* kpool = reinterpret_cast<const bf16*>(a.k_pool);
  const bf16* vpool = reinterpret_cast<const bf16*>(a.v_pool);
  for (int k0 = kbeg; k0 < kend; k0 += kKeys) {
    const int nk = min(kKeys, kend - k0);
    // Stage K (row-major) and V (transposed) for 32 keys: 16-byte chunks of 8 dims.
    for (int idx = tid; idx < kKeys * (D / 8); idx += kThreads) {
      const int kk = idx / (D / 8), d8 = (idx % (D / 8)) * 8;
      bf16x8 kh, vh, kl, vl;
      if (kk < nk) {
        const int t = k0 + kk;
        if (is_block) {
          const long long off = ((long long)(b * kBlock + t) * nkv + g) * D + d8;
          const f32x4 k0v = *reinterpret_cast<const f32x4*>(a.bk + off);
          const f32x4 k1v = *reinterpret_cast<const f32x4*>(a.bk + off + 4);
          const f32x4 v0v = *reinterpret_cast<const f32x4*>(a.bv + off);
          const f32x4 v1v = *reinterpret_cast<const f32x4*>(a.bv + off + 4);
          const float kf[8] = {k0v[0], k0v[1], k0v[2], k0v[3], k1v[0], k1v[1], k1v[2], k1v[3]};
          const float vf[8] = {v0v[0], v0v[1], v0v[2], v0v[3], v1v[0], v1v[1], v1v[2], v1v[3]};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            bf16 h1, l1, h2, l2;
            split2(kf[i], h1, l1);
            split2(vf[i], h2, l2);
            kh[i] = h1;
            kl[i] = l1;
            vh[i] = h2;
            vl[i] = l2;
          }
        } else {
          const int page = a.block_table[(long long)b * a.max_pages + t / kPage];
          const long long off = (((long long)page * nkv + g) * kPage + t % kPage) * D + d8;
          kh = *reinterpret_cast<const bf16x8*>(kpool + off);
          vh = *reinterpret_cast<const bf16x8*>(vpool + off);
#pragma unroll
          for (int i = 0; i < 8; ++i) kl[i] = vl[i] = (bf16)0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kh[i] = vh[i] = kl[i] = vl[i] = (bf16)0.f;
      }
      *reinterpret_cast<bf16x8*>(&sm.k[0][kk][d8]) = kh;
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.vt[0][d8 + i][kk] = vh[i];
      if (is_block) {
        *reinterpret_cast<bf16x8*>(&sm.k[1][kk][d8]) = kl;
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.vt[1][d8 + i][kk] = vl[i];
      }
    }
    __syncthreads();

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (wave + 4 * rt >= G) continue;
      // S = Q K^T for two 16-key tiles.
      f32x4 s[2];
#pragma unroll
      for (int kt2 = 0; kt2 < 2; ++kt2) {
        s[kt2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          for (int pb = 0; pb < npieces; ++pb) {
            const i32x4 kb = *reinterpret_cast<const i32x4*>(
                &sm.k[pb][kt2 * 16 + (lane & 15)][ks * 32 + (lane >> 4) * 8]);
            s[kt2] = mfma_tile<bf16>(qf[rt][ks][0], kb, s[kt2]);
            if (pb == 0) s[kt2] = mfma_tile<bf16>(qf[rt][ks][1], kb, s[kt2]);
          }
        }
      }
      // Online softmax over the 32 keys.  Lane holds rows 4*(lane/16)+i, key lane%16 of
      // each tile; a row's keys are the 16 lanes sharing lane/16.
      float corr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v0 = (lane & 15) < nk, v1 = 16 + (lane & 15) < nk;
        float x0 = v0 ? s[0][i] : -INFINITY, x1 = v1 ? s[1][i] : -INFINITY;
        float mx = fmaxf(x0, x1);
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
        const float mnew = fmaxf(mrow[rt][i], mx);
        const float p0 = v0 ? expf(x0 - mnew) : 0.f, p1 = v1 ? expf(x1 - mnew) : 0.f;
        float ps = p0 + p1;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, kWave);
        corr[i] = expf(mrow[rt][i] - mnew);
        lrow[rt][i] = lrow[rt][i] * corr[i] + ps;
        mrow[rt][i] = mnew;
        sm.p[wave][(lane >> 4) * 4 + i][lane & 15] = p0;
        sm.p[wave][(lane >> 4) * 4 + i][16 + (lane & 15)] = p1;
      }
      // o (rows 4*(lane/16)+i) *= corr
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[rt][dt][i] *= corr[i];
      // The probability tile is written and read back by the same wave (transpose of the
      // MFMA output layout into the A-operand layout): order the LDS accesses.
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // P as the A operand: lane holds row lane%16, keys 8*(lane/16) .. +8, split hi/lo.
      i32x4 pa[2];
      {
        bf16x8 h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 hb, lb;
          split2(sm.p[wave][lane & 15][(lane >> 4) * 8 + e], hb, lb);
          h[e] = hb;
          l[e] = lb;
        }
        pa[0] = __builtin_bit_cast(i32x4, h);
        pa[1] = __builtin_bit_cast(i32x4, l);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        for (int pb = 0; pb < npieces; ++pb) {
          const i32x4 vb = *reinterpret_cast<const i32x4*>(
              &sm.vt[pb][dt * 16 + (lane & 15)][(lane >> 4) * 8]);
          o[rt][dt] = mfma_tile<bf16>(pa[0], vb, o[rt][dt]);
          if (pb == 0) o[rt][dt] = mfma_tile<bf16>(pa[1], vb, o[rt][dt]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    __syncthreads();
  }

  // Partial of this chunk: rows r = head*16 + slot.
  const long long slot = ((long long)b * nkv + g) * (a.nc + 1) + c;
  constexpr int R = G * 16;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int hh = wave + 4 * rt;
    if (hh >= G) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = hh * 16 + (lane >> 4) * 4 + i;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        a.part_o[(slot * R + row) * D + dt * 16 + (lane & 15)] = o[rt][dt][i];
      if ((lane & 15) == 0) {
        a.part_ml[(slot * R + row) * 2 + 0] = mrow[rt][i];
        a.part_ml[(slot * R + row) * 2 + 1] = lrow[rt][i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// fp32: VALU partial kernel (rows r = head*16 + slot)
// ------------------------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(kThreads) void attn_partial_f32(AttnArgs a) {
  constexpr int G = R / kBlock;
  constexpr int OPH = kThreads / D;
  constexpr int NRO = R / OPH;
  constexpr int SPH = kThreads / kKeys;
  constexpr int NRS = R / SPH;
  __shared__ float q_s[R][D + 1];
  __shared__ float k_s[kKeys][D + 1];
  __shared__ float v_s[kKeys][D];
  __shared__ float p_s[R][kKeys + 1];
  __shared__ float m_s[R], l_s[R], sc_s[R];

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
    kbeg = (int)min((long long)c * a.chunk, (long long)T_b);
    kend = min(kbeg + a.chunk, T_b);
  }
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, i = idx % D;
    const int hh = r / kBlock, j = r % kBlock;
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

  const float* kpool = reinterpret_cast<const float*>(a.k_pool);
  const float* vpool = reinterpret_cast<const float*>(a.v_pool);
  for (int k0 = kbeg; k0 < kend; k0 += kKeys) {
    const int nk = min(kKeys, kend - k0);
    for (int idx = tid; idx < kKeys * D; idx += kThreads) {
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
          kv = kpool[off];
          vv = vpool[off];
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
      for (int n = 0; n < NRS; ++n) p_s[r0 + n * SPH][cc] = cc < nk ? s[n] : -INFINITY;
    }
    __syncthreads();
    if (tid < R) {
      const float mold = m_s[tid];
      float mx = mold;
      for (int cc = 0; cc < nk; ++cc) mx = fmaxf(mx, p_s[tid][cc]);
      const float sc = expf(mold - mx);
      float l = l_s[tid] * sc;
      for (int cc = 0; cc < kKeys; ++cc) {
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
        for (int cc = 0; cc < kKeys; ++cc) acc += p_s[r][cc] * v_s[cc][i];
        o[n] = acc;
      }
    }
    __syncthreads();
  }
  const long long slot = ((long long)b * nkv + g) * (a.nc + 1) + c;
  const int i = tid % D, r0 = tid / D;
#pragma unroll
  for (int n = 0; n < NRO; ++n) {
    const int r = r0 + n * OPH;
    a.part_o[(slot * R + r) * D + i] = o[n];
  }
  if (tid < R) {
    a.part_ml[(slot * R + tid) * 2 + 0] = m_s[tid];
    a.part_ml[(slot * R + tid) * 2 + 1] = l_s[tid];
  }
}

// ------------------------------------------------------------------------------------------
// Merge: one workgroup per (query head, request).  First the per-row maximum and total sum
// over chunks (16 threads per row, fixed order), kept as per-chunk weights in LDS; then
// every output element is the weighted sum of the chunk partials, chunks in order.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge(AttnArgs a) {
  __shared__ float w_s[kAttnMaxChunks + 1][kBlock];
  __shared__ float red[kThreads / kBlock][kBlock];
  __shared__ float M_s[kBlock], L_s[kBlock];
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.n_q / a.n_kv;
  const int g = h / G, hh = h % G;
  const int R = G * kBlock;
  const int nch = a.nc + 1;
  const long long slot0 = ((long long)b * a.n_kv + g) * nch;
  const int tid = threadIdx.x;
  const int j = tid % kBlock, lanec = tid / kBlock;        // row, chunk lane (16 lanes)
  const int r = hh * kBlock + j;

  float mx = -INFINITY;
  for (int c = lanec; c < nch; c += kThreads / kBlock) {
    const float l = a.part_ml[((slot0 + c) * R + r) * 2 + 1];
    if (l > 0.f) mx = fmaxf(mx, a.part_ml[((slot0 + c) * R + r) * 2 + 0]);
  }
  red[lanec][j] = mx;
  __syncthreads();
  if (tid < kBlock) {
    float M = -INFINITY;
    for (int q = 0; q < kThreads / kBlock; ++q) M = fmaxf(M, red[q][tid]);
    M_s[tid] = M;
  }
  __syncthreads();
  const float M = M_s[j];
  float lsum = 0.f;
  for (int c = lanec; c < nch; c += kThreads / kBlock) {
    const float l = a.part_ml[((slot0 + c) * R + r) * 2 + 1];
    const float w = l > 0.f ? expf(a.part_ml[((slot0 + c) * R + r) * 2 + 0] - M) : 0.f;
    w_s[c][j] = w;
    lsum += l * w;
  }
  red[lanec][j] = lsum;
  __syncthreads();
  if (tid < kBlock) {
    float L = 0.f;
    for (int q = 0; q < kThreads / kBlock; ++q) L += red[q][tid];
    L_s[tid] = 1.0f / L;
  }
  __syncthreads();
  for (int idx = tid; idx < kBlock * D; idx += kThreads) {
    const int jj = idx / D, i = idx % D;
    const int rr = hh * kBlock + jj;
    const float* src = a.part_o + (slot0 * R + rr) * D + i;
    const long long cstride = (long long)R * D;
    float acc = 0.f;
#pragma unroll 4
    for (int c = 0; c < nch; ++c) acc += w_s[c][jj] * src[c * cstride];
    a.out[(long long)(b * kBlock + jj) * (a.n_q * D) + h * D + i] = acc * L_s[jj];
  }
}

// ------------------------------------------------------------------------------------------
// Launch
// ------------------------------------------------------------------------------------------
static hipError_t launch_partial(int bf16_dtype, const AttnArgs& a, int batch,
                                 hipStream_t stream) {
  dim3 grid(a.nc + 1, a.n_kv, batch);
  const int G = a.n_q / a.n_kv;
  if (bf16_dtype) {
    if (a.head_dim == 128) {
      if (G == 2) attn_partial_bf16<128, 2><<<grid, kThreads, 0, stream>>>(a);
      else if (G == 4) attn_partial_bf16<128, 4><<<grid, kThreads, 0, stream>>>(a);
      else if (G == 8) attn_partial_bf16<128, 8><<<grid, kThreads, 0, stream>>>(a);
      else return hipErrorInvalidValue;
    } else if (a.head_dim == 64) {
      if (G == 2) attn_partial_bf16<64, 2><<<grid, kThreads, 0, stream>>>(a);
      else if (G == 4) attn_partial_bf16<64, 4><<<grid, kThreads, 0, stream>>>(a);
      else if (G == 8) attn_partial_bf16<64, 8><<<grid, kThreads, 0, stream>>>(a);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    const int R = G * kBlock;
    if (a.head_dim == 128) {
      if (R == 32) attn_partial_f32<128, 32><<<grid, kThreads, 0, stream>>>(a);
      else if (R == 64) attn_partial_f32<128, 64><<<grid, kThreads, 0, stream>>>(a);
      else return hipErrorInvalidValue;
    } else if (a.head_dim == 64) {
      if (R == 32) attn_partial_f32<64, 32><<<grid, kThreads, 0, stream>>>(a);
      else if (R == 64) attn_partial_f32<64, 64><<<grid, kThreads, 0, stream>>>(a);
      else if (R == 128) attn_partial_f32<64, 128><<<grid, kThreads, 0, stream>>>(a);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_block_attention(int bf16_dtype, const AttnArgs& a, int batch,
                                  hipStream_t stream) {
  hipError_t e = launch_partial(bf16_dtype, a, batch, stream);
  if (e != hipSuccess) return e;
  dim3 grid(a.n_q, batch);
  if (a.head_dim == 128) attn_merge<128><<<grid, kThreads, 0, stream>>>(a);
  else attn_merge<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

bool block_attention_supported(int bf16_dtype, int head_dim, int group) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (group != 2 && group != 4 && group != 8) return false;
  return bf16_dtype || !(head_dim == 128 && group == 8);  // fp32 kernel: LDS limit
}

}  // namespace dflash
