// Block attention of the DFlash draft pass: the 16 block queries of every head of one KV
// group attend, without a mask, to the request's injected context (paged KV cache) and to
// the 16 block keys.
//
// Pass 1 (partials), grid (nc, n_kv, batch): workgroup c covers context keys
// [c*chunk, min((c+1)*chunk, T_b)) (chunk a multiple of 32, at most 1024, fixed by the
// caller, so the page ids of a chunk are one load per lane issued before T_b arrives), and
// the last workgroup also the 16 block keys (so a grid of nc * n_kv * batch workgroups fills
// the chip in one round).  One wave per query head of the KV group.  Each wave keeps an
// online softmax (running max m, sum l, unnormalized output o) and writes (m, l, o).
// Pass 2 (merge), grid (n_q, d / 32, batch): rescales the nc partials of each head to a
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
// No LDS and no barriers.  Cache K/V are exact bf16 operands; fp32 queries, probabilities
// and block keys/values enter as hi + lo bf16 pairs (the lo x lo product, ~2^-32 relative,
// is dropped).  fp32 models use a VALU version of pass 1 with the same partial layout.
//
// Partial layout: part_o[slot][head_in_group][dt][q][row][i] holds output dim
// 16*dt + 4*q + i of block row `row` (a float4 per (dt, q, row)); part_ml[slot][head][row]
// holds (m, l).  slot = (b * n_kv + g) * nc + c.
#include "attention.h"
#include "common.h"

namespace dflash {

typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ inline long long part_o_index(long long slot, int G, int hh, int D, int row,
                                         int dim) {
  return ((((slot * G + hh) * (D / 16) + dim / 16) * 4 + (dim % 16) / 4) * kBlock + row) * 4 +
         dim % 4;
}

__device__ inline void split2(float v, bf16& hi, bf16& lo) {
  hi = (bf16)v;
  lo = (bf16)(v - (float)hi);
}

// 8 floats -> hi and lo bf16 fragments.
__device__ inline void split8(const float (&f)[8], i32x4& hi, i32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16 hb, lb;
    split2(f[i], hb, lb);
    h[i] = hb;
    l[i] = lb;
  }
  hi = __builtin_bit_cast(i32x4, h);
  lo = __builtin_bit_cast(i32x4, l);
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
// bf16: MFMA partial kernel, one wave per query head of the group
// ------------------------------------------------------------------------------------------
template <int D>
struct StepRegs {
  i32x4 k[2][D / 32];      // two pages x dim steps
  i32x2 v[D / 16][2];      // dim tiles x pages
  int nk;                  // valid keys of the step (1..32)
};

template <int D, int G>
__global__ __launch_bounds__(G * kWave, 2) void attn_partial_bf16(AttnArgs a) {
  constexpr int KS = D / 32;                  // dim steps of S^T
  constexpr int DT = D / 16;                  // dim tiles of O^T
  constexpr int kBlockBytes = kBlock * D * 4; // the block's K, or its V^T, in fp32
  constexpr int kCopies = 2 * kBlockBytes / 1024;   // 1 KB (64 lanes x 16 B) per copy
  static_assert(kCopies % G == 0, "block copies split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char blk_s[2 * kBlockBytes];   // K, then V^T
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, hh = threadIdx.x / kWave;
  const int n = lane & 15, q = lane >> 4;
  const int nq = a.n_q, nkv = a.n_kv;
  // Physical page ids of the chunk's (at most 64) logical pages (lane i: page i), fetched
  // together with T_b; indices are clamped into the table row.
  const int kbeg0 = c * a.chunk;
  const int* table = a.block_table + (long long)b * a.max_pages;
  const int pid = table[min(kbeg0 / kPage + lane, a.max_pages - 1)];
  const int T_b = a.ctx_lens[b];
  const bool has_block = c == a.nc - 1;
  const int kbeg = min(kbeg0, T_b);
  const int kend = min(kbeg0 + a.chunk, T_b);

  // The last chunk's workgroup copies the block's fp32 keys [16][d] and transposed values
  // [d][16] (contiguous per KV group) into LDS with direct loads, which need no registers.
  // The other workgroups issue the same copies from the first kilobyte of the arrays (and
  // never read them), so that every wave's load count is the same on every path.
  {
    const long long grp = has_block ? (long long)(b * nkv + g) * kBlockBytes : 0;
    const char* srck = reinterpret_cast<const char*>(a.bk) + grp;
    const char* srcv = reinterpret_cast<const char*>(a.bv) + grp;
#pragma unroll
    for (int j = 0; j < kCopies / G; ++j) {
      const int i = hh + j * G;
      const int half = i / (kCopies / 2), off = (i % (kCopies / 2)) * 1024;
      const char* src = (half ? srcv : srck) + (has_block ? off : 0) + lane * 16;
      __builtin_amdgcn_global_load_lds((global_void_ptr)src,
                                       (lds_void_ptr)(blk_s + half * kBlockBytes + off), 16, 0,
                                       0);
    }
  }
  // Issue all of the above before the page ids are waited for (the compiler waits for every
  // outstanding load once a direct-to-LDS load is pending, so that first wait retires them).
  __builtin_amdgcn_sched_barrier(0);

  // Q^T rows of this head (B operand of S^T): lane holds block row n, dims 32*ks + 8q .. +8.
  f32x4 qraw[KS][2];
  {
    const float* src = a.q + ((long long)(b * kBlock + n) * nq + g * G + hh) * D + q * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qraw[ks][0] = *reinterpret_cast<const f32x4*>(src + ks * 32);
      qraw[ks][1] = *reinterpret_cast<const f32x4*>(src + ks * 32 + 4);
    }
  }

  const bf16* kpool = reinterpret_cast<const bf16*>(a.k_pool);
  const bf16* vpool = reinterpret_cast<const bf16*>(a.v_pool);
  const int npg = (kend - kbeg + kPage - 1) / kPage;   // 0..64 (chunk <= 1024 keys)
  const int nsteps = (kend - kbeg + 31) / 32;
  // Step st reads logical pages 2st and 2st+1 of the chunk, whose physical ids lanes 2st
  // and 2st+1 of `pid` hold; a page past the chunk's last is read from the last one (its
  // keys are masked).  Every step issues the same loads with no branch, so the compiler
  // can wait for one step's loads while the next step's stay in flight.
  const int pid_safe = npg > 0 ? pid : 0;
  auto load_step = [&](int st, StepRegs<D>& r) {
    r.nk = min(32, kend - kbeg - 32 * st);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const long long page =
          __builtin_amdgcn_readlane(pid_safe, max(min(2 * st + pg, npg - 1), 0));
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
  load_step(min(1, max(nsteps - 1, 0)), rb);
  __builtin_amdgcn_sched_barrier(0);   // keep every prologue load ahead of the math below

  // Q^T fragments, scaled by log2(e) / sqrt(d) and split hi/lo.
  i32x4 qf[KS][2];
  const float qscale = a.scale * kLog2e;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const f32x4 v0 = qraw[ks][0] * qscale, v1 = qraw[ks][1] * qscale;
    const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    split8(f, qf[ks][0], qf[ks][1]);
  }

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Online-softmax update for one 32-key step given S^T tiles s[2] (lane: keys
  // 16 pg + 4q + i for query n); returns the P^T fragment (hi, lo).  The accumulator is
  // rescaled only when some row's maximum grew (a branch uniform over the wave).
  auto softmax_step = [&](const f32x4 (&s)[2], int nk, i32x4& p_hi, i32x4& p_lo) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e / 4][e % 4];
    if (nk < 32) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (16 * (e / 4) + 4 * q + e % 4 >= nk) x[e] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    const float m_new = fmaxf(m_run, rows_max(mx));   // finite: key 0 of a step is valid
    if (__ballot(m_new > m_run)) {
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first step
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    float pv[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
    if (nk < 32) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (16 * (e / 4) + 4 * q + e % 4 >= nk) pv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ps += pv[e];
    l_run += rows_sum(ps);
    split8(pv, p_hi, p_lo);
  };

  auto compute_step = [&](const StepRegs<D>& r) {
    // Q hi and Q lo products accumulate separately: four independent MFMA chains.
    f32x4 sh[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 sl[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        sh[pg] = mfma_tile<bf16>(r.k[pg][ks], qf[ks][0], sh[pg]);
        sl[pg] = mfma_tile<bf16>(r.k[pg][ks], qf[ks][1], sl[pg]);
      }
    const f32x4 s[2] = {sh[0] + sl[0], sh[1] + sl[1]};
    i32x4 ph, pl;
    softmax_step(s, r.nk, ph, pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      i32x4 v = i32x4{r.v[dt][0][0], r.v[dt][0][1], r.v[dt][1][0], r.v[dt][1][1]};
      if (r.nk < 32) v = mask_vt(v, q, r.nk);   // stale cache slots may hold any bits
      o[dt] = mfma_tile<bf16>(v, ph, o[dt]);
      o[dt] = mfma_tile<bf16>(v, pl, o[dt]);
    }
  };
  // Steady state: ra holds step st, rb step st + 1, and both prefetches exist.
  int st = 0;
  for (; st + 3 < nsteps; st += 2) {
    compute_step(ra);
    load_step(st + 2, ra);
    compute_step(rb);
    load_step(st + 3, rb);
  }
  // 0..3 steps remain.
  if (st < nsteps) compute_step(ra);
  if (st + 2 < nsteps) load_step(st + 2, ra);
  if (st + 1 < nsteps) compute_step(rb);
  if (st + 2 < nsteps) compute_step(ra);

  if (has_block) {   // the 16 block keys, hi + lo on both operands, from LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const float* bk_s = reinterpret_cast<const float*>(blk_s);
    const float* bv_s = reinterpret_cast<const float*>(blk_s + kBlockBytes);
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(bk_s + n * D + ks * 32 + q * 8);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(bk_s + n * D + ks * 32 + q * 8 + 4);
      const float f[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      i32x4 kh, kl;
      split8(f, kh, kl);
      s[0] = mfma_tile<bf16>(kh, qf[ks][0], s[0]);
      s[0] = mfma_tile<bf16>(kh, qf[ks][1], s[0]);
      s[0] = mfma_tile<bf16>(kl, qf[ks][0], s[0]);
    }
    i32x4 ph, pl;
    softmax_step(s, kBlock, ph, pl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 vv = *reinterpret_cast<const f32x4*>(bv_s + (16 * dt + n) * kBlock + q * 4);
      const float f[8] = {vv[0], vv[1], vv[2], vv[3], 0.f, 0.f, 0.f, 0.f};
      i32x4 vh, vl;
      split8(f, vh, vl);
      o[dt] = mfma_tile<bf16>(vh, ph, o[dt]);
      o[dt] = mfma_tile<bf16>(vh, pl, o[dt]);
      o[dt] = mfma_tile<bf16>(vl, ph, o[dt]);
    }
  }

  // Partial of this chunk.  O^T layout: lane holds dims 16dt + 4q + i of block row n.
  const long long slot = ((long long)b * nkv + g) * a.nc + c;
  f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + (slot * G + hh) * (DT * 4 * kBlock);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) po[(dt * 4 + q) * kBlock + n] = o[dt];
  if (q == 0) {
    float* ml = a.part_ml + ((slot * G + hh) * kBlock + n) * 2;
    ml[0] = m_run;
    ml[1] = l_run;
  }
}

// ------------------------------------------------------------------------------------------
// fp32: VALU partial kernel (rows r = head*16 + slot)
// ------------------------------------------------------------------------------------------
constexpr int kKeys = 32;       // keys per step
constexpr int kThreads = 256;   // 4 waves

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
  const bool has_block = c == a.nc - 1;
  const float qscale = a.scale * kLog2e;   // base-2 scores, as in the MFMA kernel
  const int kbeg = min(c * a.chunk, T_b);
  const int kend = min(kbeg + a.chunk, T_b);
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, i = idx % D;
    const int hh = r / kBlock, j = r % kBlock;
    q_s[r][i] = a.q[((long long)(b * kBlock + j) * nq + g * G + hh) * D + i] * qscale;
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
  // Context steps of 32 keys, then (last workgroup) one step over the 16 block keys.
  const int n_ctx_steps = (kend - kbeg + kKeys - 1) / kKeys;
  for (int st = 0; st < n_ctx_steps + (has_block ? 1 : 0); ++st) {
    const bool is_block = st == n_ctx_steps;
    const int k0 = is_block ? 0 : kbeg + st * kKeys;
    const int nk = is_block ? kBlock : min(kKeys, kend - k0);
    for (int idx = tid; idx < kKeys * D; idx += kThreads) {
      const int kk = idx / D, i = idx % D;
      float kv = 0.f, vv = 0.f;
      if (kk < nk) {
        const int t = k0 + kk;
        if (is_block) {
          kv = a.bk[((long long)(b * nkv + g) * kBlock + t) * D + i];
          vv = a.bv[((long long)(b * nkv + g) * D + i) * kBlock + t];
        } else {
          const long long page = a.block_table[(long long)b * a.max_pages + t / kPage];
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
      for (int n = 0; n < NRS; ++n) p_s[r0 + n * SPH][cc] = cc < nk ? s[n] : -INFINITY;
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
  const long long slot = ((long long)b * nkv + g) * a.nc + c;
  const int i = tid % D, r0 = tid / D;
#pragma unroll
  for (int n = 0; n < NRO; ++n) {
    const int r = r0 + n * OPH;
    a.part_o[part_o_index(slot, G, r / kBlock, D, r % kBlock, i)] = o[n];
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
// result is written in the fragment layout the output projection reads.
// ------------------------------------------------------------------------------------------
constexpr int kMergeBatch = 40;
constexpr int kMergeThreads = 128;   // float4s of a 16 x 32 slice

template <int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge(AttnArgs a) {
  constexpr int NCL = kMergeThreads / kBlock;   // chunk lanes per row
  constexpr int NT = D * 4;                     // float4s of one head's 16 x D partial
  __shared__ float w_s[kAttnMaxChunks + 1][kBlock];
  __shared__ float m_s[kAttnMaxChunks + 1][kBlock];
  __shared__ float red[NCL][kBlock];
  __shared__ float M_s[kBlock], invL_s[kBlock];
  const int h = blockIdx.x, slice = blockIdx.y, b = blockIdx.z;
  const int G = a.n_q / a.n_kv;
  const int g = h / G, hh = h % G;
  const int nch = a.nc;
  const long long slot0 = ((long long)b * a.n_kv + g) * nch;
  const int tid = threadIdx.x;
  const int f = slice * kMergeThreads + tid;     // float4 index (dt, q, row) within the head
  const long long cstride = (long long)G * NT;   // float4s between chunks
  const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o) + (slot0 * G + hh) * NT + f;

  f32x4 v[kMergeBatch];
#pragma unroll
  for (int c = 0; c < kMergeBatch; ++c)
    v[c] = c < nch ? src[c * cstride] : f32x4{0.f, 0.f, 0.f, 0.f};

  // Row maximum and weights.  Thread (row j, chunk lane cl).
  const int j = tid % kBlock, cl = tid / kBlock;
  float mx = -INFINITY;
  for (int c = cl; c < nch; c += NCL) {
    const float* ml = a.part_ml + (((slot0 + c) * G + hh) * kBlock + j) * 2;
    const float m = ml[0], l = ml[1];
    const float mm = l > 0.f ? m : -INFINITY;   // empty chunks carry no weight
    m_s[c][j] = mm;
    w_s[c][j] = l;
    mx = fmaxf(mx, mm);
  }
  red[cl][j] = mx;
  __syncthreads();
  if (tid < kBlock) {
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
  if (tid < kBlock) {
    float L = 0.f;
    for (int r = 0; r < NCL; ++r) L += red[r][tid];
    invL_s[tid] = 1.0f / L;
  }
  __syncthreads();

  // float4 f = (dt, q, row): row f % 16, dims 16*(f/64) + 4*((f/16)%4) .. +3.
  const int row = f % kBlock;
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
  const int dim = 16 * (f / (4 * kBlock)) + 4 * ((f / kBlock) % 4);
  const int kto = a.n_q * D / (4 * a.out_kper);
  *reinterpret_cast<f32x4*>(a.out + swz_off(b * kBlock + row, h * D + dim, kto, a.out_kper)) =
      acc * invL_s[row];
}

// ------------------------------------------------------------------------------------------
// Launch
// ------------------------------------------------------------------------------------------
template <int D>
static void launch_partial_bf16(int G, dim3 grid, const AttnArgs& a, hipStream_t stream) {
  switch (G) {
    case 1: attn_partial_bf16<D, 1><<<grid, 1 * kWave, 0, stream>>>(a); break;
    case 2: attn_partial_bf16<D, 2><<<grid, 2 * kWave, 0, stream>>>(a); break;
    case 4: attn_partial_bf16<D, 4><<<grid, 4 * kWave, 0, stream>>>(a); break;
    case 8: attn_partial_bf16<D, 8><<<grid, 8 * kWave, 0, stream>>>(a); break;
    default: break;
  }
}

static hipError_t launch_partial(int bf16_dtype, const AttnArgs& a, int batch,
                                 hipStream_t stream) {
  dim3 grid(a.nc, a.n_kv, batch);
  const int G = a.n_q / a.n_kv;
  if (!block_attention_supported(bf16_dtype, a.head_dim, G)) return hipErrorInvalidValue;
  if (bf16_dtype) {
    if (a.head_dim == 128) launch_partial_bf16<128>(G, grid, a, stream);
    else launch_partial_bf16<64>(G, grid, a, stream);
  } else {
    const int R = G * kBlock;
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

hipError_t launch_block_attention(int bf16_dtype, const AttnArgs& a, int batch,
                                  hipStream_t stream) {
  if (a.nc < 1 || a.nc > kAttnMaxChunks || a.chunk < 32 || a.chunk % 32 ||
      a.chunk > kAttnMaxChunkKeys)
    return hipErrorInvalidValue;
  hipError_t e = launch_partial(bf16_dtype, a, batch, stream);
  if (e != hipSuccess) return e;
  dim3 grid(a.n_q, a.head_dim / 32, batch);
  if (a.head_dim == 128) attn_merge<128><<<grid, kMergeThreads, 0, stream>>>(a);
  else attn_merge<64><<<grid, kMergeThreads, 0, stream>>>(a);
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
