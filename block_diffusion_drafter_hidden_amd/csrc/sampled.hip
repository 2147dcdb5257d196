// Temperature-1 verification: speculative accept/reject with residual resampling.
//
// Kernel 1, one workgroup per (request, row) over the 15 draft rows and 16 target rows:
// softmax statistics (row max, sum of exp(x - max)) and, for draft rows, the inverse-CDF
// draw of the draft token.  Kernel 2, one workgroup per request: the sequential accept test
// over the 15 drafts (scalar reads of the statistics), then one inverse-CDF draw from the
// residual max(0, p - q) at the first rejection, or from p_16 if every draft is accepted.
//
// Inverse CDF over a row of V weights: each of the 256 threads owns a contiguous segment;
// segment sums, an exclusive prefix over segments in thread order, then the segment that
// crosses u * total is scanned element by element.  All sums run in a fixed order.
//
// Weights exp(x - max), sums, the accept test and the residual are evaluated in fp64: with
// a 128k vocabulary one token's share of the mass is ~1e-5, so fp32 running sums (relative
// error ~1e-6) would move the sampled index; fp64 keeps every decision the same as an fp64
// evaluation of the rule up to ~1e-13 of the mass.
#include "common.h"
#include "sampled.h"

namespace dflash {

constexpr int kThr = 256;
constexpr int kRows = 2 * kDrafts + 1;  // 15 draft rows + 16 target rows

struct RowScan {
  double seg[kThr];
  double pre[kThr];
  float red[kThr];
  double dred[kThr];
  int pick;
  double total;
};

// Inverse CDF of weights w(v) (v in [0, V)) at u: smallest j with cumsum(w)[j] > u * sum(w),
// else the last j with w(j) > 0.  The running sum is the exclusive prefix of the segment
// sums plus a wave-level inclusive scan inside the segment, always in the same order.
// Must be called by all threads; returns the index to all.
template <typename W>
__device__ int inv_cdf_row(W w, int V, float u, RowScan& sh, double* total_out) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int seg_len = (V + kThr - 1) / kThr;
  {
    const int s0 = min(tid * seg_len, V), s1 = min(s0 + seg_len, V);
    double s = 0.0;
    for (int v = s0; v < s1; ++v) s += w(v);
    sh.seg[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < kThr; ++t) {
      sh.pre[t] = run;
      run += sh.seg[t];
    }
    sh.total = run;
  }
  __syncthreads();
  const double total = sh.total;
  const double thr = (double)u * total;
  if (tid < kWave) {
    int t0 = kThr - 1;
    for (int t = 0; t < kThr; ++t)
      if (sh.pre[t] + sh.seg[t] > thr) {
        t0 = t;
        break;
      }
    int pick = -1;
    for (int t = t0; t < kThr && pick < 0; ++t) {
      const int a0 = min(t * seg_len, V), a1 = min(a0 + seg_len, V);
      double base = sh.pre[t];
      for (int c0 = a0; c0 < a1 && pick < 0; c0 += kWave) {
        const int v = c0 + lane;
        double x = v < a1 ? w(v) : 0.0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const double y = __shfl_up(x, o, kWave);
          if (lane >= o) x += y;
        }
        const unsigned long long hit = __ballot(v < a1 && base + x > thr);
        if (hit) pick = c0 + __ffsll((long long)hit) - 1;
        base += __shfl(x, kWave - 1, kWave);
      }
    }
    for (int c1 = V; c1 > 0 && pick < 0; c1 -= kWave) {
      const int v = c1 - kWave + lane;
      const unsigned long long pos = __ballot(v >= 0 && w(v) > 0.0);
      if (pos) pick = c1 - kWave + (63 - __clzll((long long)pos));
    }
    if (lane == 0) sh.pick = pick < 0 ? 0 : pick;
  }
  __syncthreads();
  if (total_out) *total_out = total;
  const int r = sh.pick;
  __syncthreads();
  return r;
}

__device__ float block_max(float v, float* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = kThr / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ double block_sum_fixed(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = kThr / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = red[tid] + red[tid + o];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThr) void sampled_stats_kernel(SampledArgs a) {
  __shared__ RowScan sh;
  const int row = blockIdx.x;  // 0..14 draft rows, 15..30 target rows
  const int b = blockIdx.y;
  const int V = a.vocab;
  const bool is_draft = row < kDrafts;
  const float* x = is_draft ? a.draft_logits + ((long long)b * kDrafts + row) * V
                            : a.target_logits + ((long long)b * kBlock + (row - kDrafts)) * V;
  float m = -INFINITY;
  for (int v = threadIdx.x; v < V; v += kThr) m = fmaxf(m, x[v]);
  m = block_max(m, sh.red);
  const double md = m;
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += kThr) s += exp((double)x[v] - md);
  s = block_sum_fixed(s, sh.dred);
  if (threadIdx.x == 0) {
    a.stats[((long long)b * kRows + row) * 2 + 0] = md;
    a.stats[((long long)b * kRows + row) * 2 + 1] = s;
  }
  if (is_draft) {
    const float u = a.u_draft[(long long)b * kDrafts + row];
    auto w = [=](int v) { return exp((double)x[v] - md); };
    const int d = inv_cdf_row(w, V, u, sh, nullptr);
    if (threadIdx.x == 0) a.draft_ids[(long long)b * kDrafts + row] = d;
  }
}

__global__ __launch_bounds__(kThr) void sampled_accept_kernel(SampledArgs a) {
  __shared__ RowScan sh;
  __shared__ int rej;
  const int b = blockIdx.x;
  const int V = a.vocab;
  const double* st = a.stats + (long long)b * kRows * 2;
  if (threadIdx.x == 0) {
    int r = kDrafts;
    for (int i = 0; i < kDrafts; ++i) {
      const int d = a.draft_ids[(long long)b * kDrafts + i];
      const float* dl = a.draft_logits + ((long long)b * kDrafts + i) * V;
      const float* tl = a.target_logits + ((long long)b * kBlock + i) * V;
      const double qd = exp((double)dl[d] - st[2 * i]) / st[2 * i + 1];
      const double pd = exp((double)tl[d] - st[2 * (kDrafts + i)]) / st[2 * (kDrafts + i) + 1];
      if (!((double)a.u_accept[(long long)b * kDrafts + i] * qd < pd)) {
        r = i;
        break;
      }
    }
    rej = r;
  }
  __syncthreads();
  const int i = rej;
  const float u = a.u_resample[b];
  int x;
  const float* tl = a.target_logits + ((long long)b * kBlock + i) * V;
  const double mp = st[2 * (kDrafts + i)], sp = st[2 * (kDrafts + i) + 1];
  if (i < kDrafts) {
    const float* dl = a.draft_logits + ((long long)b * kDrafts + i) * V;
    const double mq = st[2 * i], sq = st[2 * i + 1];
    auto res = [=](int v) {
      return fmax(exp((double)tl[v] - mp) / sp - exp((double)dl[v] - mq) / sq, 0.0);
    };
    double total;
    x = inv_cdf_row(res, V, u, sh, &total);
    if (!(total > 0.0)) {
      auto pw = [=](int v) { return exp((double)tl[v] - mp); };
      x = inv_cdf_row(pw, V, u, sh, nullptr);
    }
  } else {
    auto pw = [=](int v) { return exp((double)tl[v] - mp); };
    x = inv_cdf_row(pw, V, u, sh, nullptr);
  }
  const int t = threadIdx.x;
  if (t < kBlock) {
    int e = -1;
    if (t < i) e = a.draft_ids[(long long)b * kDrafts + t];
    else if (t == i) e = x;
    a.emitted[(long long)b * kBlock + t] = e;
  }
  if (t == 0) a.accept_len[b] = i + 1;
}

hipError_t launch_verify_sampled(const SampledArgs& a, int batch, hipStream_t stream) {
  sampled_stats_kernel<<<dim3(kRows, batch), kThr, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sampled_accept_kernel<<<batch, kThr, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace dflash
