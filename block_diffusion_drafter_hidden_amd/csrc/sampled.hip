// Temperature-1 verification: speculative accept/reject with residual resampling.
//
// A row of V logits is read in "wave chunks" of 256 consecutive elements (one wave, 16
// bytes per lane: 1 KB contiguous per load instruction).  Wave w of a workgroup takes wave
// chunks w, w + 4, ...; each chunk is reduced inside the wave (shuffles, no barrier).
//
// Kernel 1, one workgroup per (request, row) over the 15 draft rows and 16 target rows:
// the row's softmax statistics (max m, sum of exp(x - m)) in one pass, each lane summing
// against a per-wave reference (layout at kSC below).  For a draft row the sums of every
// 1024 elements are kept in LDS, and the draft token is drawn by inverse CDF: a prefix over
// those sums finds the 1024 elements that cross u * total, which one wave scans (4 KB read
// again).
// Kernel 2, kSegWG workgroups per request: each evaluates the accept tests (one lane per
// draft), finds the first rejection i and writes the chunk sums of the weights the last
// token is drawn from -- the residual max(0, p_i - q_i), or p_16 when every draft is
// accepted.  Kernel 3, one workgroup per request: the prefix over those chunk sums (staged
// in LDS) and a scan of the crossing chunk draw the token.  Every row is read once, plus 1 KB per draw;
// the rejected pair is read once more by kernel 2.
//
// Weights exp(x - m), sums, prefixes and the accept test are fp64, in a fixed order: with
// a 128k vocabulary a token's share of the mass is ~1e-5, and fp32 weights (x - m rounded,
// then exp) err by up to ~1e-6 relative, enough to move a draw into a neighbouring cell.
// exp runs as 2^((x - m) log2 e) with the exponent split off and a degree-8 Taylor polynomial
// for 2^f, |f| <= 1/2 (relative error < 4e-10).  A decision then differs from an exact
// evaluation of the rule only when u * total lies within ~1e-9 of the mass of a cumulative
// boundary, or u * q within ~1e-9 relative of p.
#include "common.h"
#include "sampled.h"

namespace dflash {

constexpr int kThr = 256;
constexpr int kWaves = kThr / kWave;
constexpr int kRows = 2 * kDrafts + 1;   // 15 draft rows + 16 target rows
constexpr int kWC = 4 * kWave;           // elements per wave chunk
constexpr int kSegWG = 32;               // workgroups per request in kernel 2

// exp(x - m) for x <= m, as 2^y with y = (x - m) log2 e formed by one fp64 fma from
// c = -m log2 e: 2^n * 2^f with n = rint(y), f = y - n in [-1/2, 1/2], and
// 2^f = sum_k (f ln 2)^k / k! to k = 8 (truncation < 2.1e-10 relative; the terms k >= 4,
// below 6.6e-4, in fp32, err by < 1.5e-10), then scaled by 2^n (ldexp, which also gives the subnormal range;
// y is clamped at -1100, where the result is 0, so x = -inf gives 0).  The fp64 constants
// (log2 e, (ln 2)^k / k! for k = 1..3) come in `k` from the kernel arguments.
constexpr double kLog2eD = 1.4426950408889634074;
__device__ inline double exp_from(float x, double c, const double (&k)[4]) {
  constexpr float c4 = 0.0096181291076284771620f, c5 = 0.0013333558146428443423f,
                  c6 = 1.5403530393381609955e-4f, c7 = 1.5252733804059840280e-5f,
                  c8 = 1.3215486790144309489e-6f;
  const double y = __builtin_fmax(fma((double)x, k[0], c), -1100.0);
  const double n = __builtin_rint(y);
  const double f = y - n;
  const float ff = (float)f;
  const float q = fmaf(fmaf(fmaf(fmaf(c8, ff, c7), ff, c6), ff, c5), ff, c4);
  const double p = fma(fma(fma(fma((double)q, f, k[3]), f, k[2]), f, k[1]), f, 1.0);
  return __builtin_ldexp(p, (int)n);
}
__device__ inline double neg_scaled(float m) { return -(double)m * kLog2eD; }

// Four elements v0 .. v0+3 of a row (v0 % 4 == 0); past V they read as -inf.
__device__ inline f32x4 load4(const float* x, int v0, int V, bool vec) {
  if (vec && v0 + 3 < V) return *reinterpret_cast<const f32x4*>(x + v0);
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = v0 + e < V ? x[v0 + e] : -INFINITY;
  return r;
}

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The first index whose inclusive prefix over n values r(k) (k = 0 .. n-1, in order),
// starting from `base`, exceeds thr; n if none.  *before gets the prefix before it (the
// whole sum plus base when none).  red must hold kWaves + 1 doubles, pick kWaves ints.  All
// threads call; all get the result.  Fixed summation order.
template <typename R>
__device__ int block_cross(R r, int n, double base, double thr, double* red, int* pick,
                           double* before) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  for (int k0 = 0; k0 < n; k0 += kThr) {
    const int k = k0 + tid;
    const double x = k < n ? r(k) : 0.0;
    double inc = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) red[w] = inc;
    __syncthreads();
    double pre = base;
    for (int i = 0; i < w; ++i) pre += red[i];
    double all = base;
    for (int i = 0; i < kWaves; ++i) all += red[i];
    const bool hit = k < n && pre + inc > thr;
    const unsigned long long bal = __ballot(hit);
    if (lane == 0) pick[w] = bal ? k0 + w * kWave + __ffsll((long long)bal) - 1 : -1;
    __syncthreads();
    int first = -1;
    for (int i = 0; i < kWaves && first < 0; ++i) first = pick[i];
    if (first >= 0) {
      // the prefix before `first`: its thread's exclusive prefix, sent through LDS
      if (k == first) red[kWaves] = pre + inc - x;
      __syncthreads();
      *before = red[kWaves];
      __syncthreads();
      return first;
    }
    __syncthreads();
    base = all;
  }
  *before = base;
  return n;
}

// One wave's inverse-CDF scan of the 256 weights of wave chunk c, lane l holding e[0..3] of
// elements v0 = 256 c + 4 l .. v0 + 3: the first j whose running sum from `base` exceeds
// thr, else the chunk's last positive weight (or -1).
__device__ int wave_scan_e(const double (&e)[4], int v0, double base, double thr) {
  const int lane = threadIdx.x % kWave;
  const double t = (e[0] + e[1]) + (e[2] + e[3]);
  double inc = t;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  double run = base + inc - t;
  int hit = -1, last = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    run += e[j];
    if (hit < 0 && run > thr && e[j] > 0.0) hit = v0 + j;
    if (e[j] > 0.0) last = v0 + j;
  }
  const unsigned long long bal = __ballot(hit >= 0);
  if (bal) return __shfl(hit, __ffsll((long long)bal) - 1, kWave);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
  return last;
}
// The same scan, loading the weights: w.four(v0, e) gives those of v0 .. v0 + 3 (0 past the
// row).
template <typename W>
__device__ int wave_scan(const W& w, int c, double base, double thr) {
  const int v0 = c * kWC + 4 * (threadIdx.x % kWave);
  double e[4];
  w.four(v0, e);
  return wave_scan_e(e, v0, base, thr);
}

// exp(x - m) of a row.
struct RowWeights {
  const float* x;
  int V;
  bool vec;
  float m;
  const double* ek;
  __device__ void four(int v0, double* e) const {
    const f32x4 v = load4(x, v0, V, vec);
    const double k = neg_scaled(m);
    const double(&kk)[4] = *reinterpret_cast<const double(*)[4]>(ek);
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = exp_from(v[j], k, kk);
  }
};

// Stats pass layout: a row is cut into super-chunks of kSC = 1024 elements; wave w takes
// super-chunks w, w + 4, ...; load j (j < 4) of a super-chunk reads its elements
// 256 j + 4 lane .. + 3 (1 KB contiguous per load).  Each lane sums exp(x - R) over its
// elements against one reference R per wave (the wave's first maximum, raised -- with the
// lane sums rescaled -- only when a value exceeds it by 2^9, so the fp64 sums never
// overflow), so no cross-lane reduction is needed until the end.  For a draft row the
// wave also reduces each super-chunk's sum and keeps it in LDS with its reference.
constexpr int kSC = 4 * kWC;
constexpr float kRaise = 512.f;

struct StatsSmem {
  float wm[kWaves], wr[kWaves];
  double ws[kWaves];
  double red[kWaves + 1];
  int pick[kWaves];
  double slice_tot[kWaves];   // the crossing super-chunk's four slice sums
  int draw;                   // the drawn draft token
};
// Dynamic LDS of the stats kernel: the super-chunks' references (floats), then their sums.
__host__ __device__ inline size_t stats_lds_bytes(int nsc) {
  return (((size_t)nsc * 4 + 7) & ~(size_t)7) + (size_t)nsc * 8;
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// At most 64 VGPRs: 8 waves per SIMD hold 8 workgroups per CU, so the 31 x 64 rows of the
// 64-request verify run in one round on 256 CUs (at 7 per CU a second, nearly empty round
// of 10% of the rows doubled the kernel's time).
__global__ __launch_bounds__(kThr) __attribute__((amdgpu_waves_per_eu(8, 8)))
void sampled_stats_kernel(SampledArgs a) {
  __shared__ StatsSmem sh;
  extern __shared__ double dyn_lds[];
  const int row = blockIdx.x;   // 0..14 draft rows, 15..30 target rows
  const int b = blockIdx.y;
  const int V = a.vocab, nsc = (V + kSC - 1) / kSC;
  const bool vec = (V & 3) == 0;
  const bool is_draft = row < kDrafts;
  const float* x = is_draft ? a.draft_logits + ((long long)b * kDrafts + row) * V
                            : a.target_logits + ((long long)b * kBlock + (row - kDrafts)) * V;
  float* sref = reinterpret_cast<float*>(dyn_lds);
  double* ssum = reinterpret_cast<double*>(reinterpret_cast<char*>(dyn_lds) +
                                           ((((size_t)nsc * 4) + 7) & ~(size_t)7));
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  float R = -INFINITY;   // this wave's reference (uniform)
  float m = -INFINITY;   // this lane's maximum
  double s = 0.0;        // this lane's sum of exp(x - R)
  auto chunk = [&](int sc, const f32x4 (&v)[4]) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lm = fmaxf(lm, fmaxf(fmaxf(v[j][0], v[j][1]), fmaxf(v[j][2], v[j][3])));
    m = fmaxf(m, lm);
    if (__ballot(lm > R + kRaise)) {   // (re)set the reference: rare after the first time
      const float Rn = wave_max_f(lm);
      s = s * exp_from(R, neg_scaled(Rn), a.exp_k);
      R = Rn;
    }
    double p = 0.0;
    if (R != -INFINITY) {   // else every value so far is -inf: weights 0
      const double k = neg_scaled(R);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p += (exp_from(v[j][0], k, a.exp_k) + exp_from(v[j][1], k, a.exp_k)) +
             (exp_from(v[j][2], k, a.exp_k) + exp_from(v[j][3], k, a.exp_k));
      s += p;
    }
    if (is_draft) {
      const double cs = wave_sum_d(p);
      if (lane == 0) {
        sref[sc] = R;
        ssum[sc] = cs;
      }
    }
  };
  // Whole super-chunks with plain 16-byte loads (non-temporal: the logits are streamed once;
  // measured 4% faster), then the row's partial last one (if any) with bounds-checked loads.
  const int nfull = vec ? V / kSC : 0;
  int sc = w;
  for (; sc < nfull; sc += kWaves) {
    const float* src = x + (long long)sc * kSC + 4 * lane;
    f32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + j * kWC));
    chunk(sc, v);
  }
  for (; sc < nsc; sc += kWaves) {
    f32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = load4(x, sc * kSC + j * kWC + 4 * lane, V, vec);
    chunk(sc, v);
  }
  {  // the wave's maximum and sum (against R), then the row's (max, sum)
    const float wmax = wave_max_f(m);
    const double wsum = wave_sum_d(s);
    if (lane == 0) {
      sh.wm[w] = wmax;
      sh.wr[w] = R;
      sh.ws[w] = wsum;
    }
  }
  __syncthreads();
  float M = sh.wm[0];
  for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sh.wm[i]);
  double S = 0.0;
  for (int i = 0; i < kWaves; ++i)
    if (sh.wr[i] != -INFINITY) S += sh.ws[i] * exp_from(sh.wr[i], neg_scaled(M), a.exp_k);
  if (threadIdx.x == 0) {
    a.stats[((long long)b * kRows + row) * 2 + 0] = (double)M;
    a.stats[((long long)b * kRows + row) * 2 + 1] = S;
  }
  if (!is_draft) return;
  // Draw the draft token: the super-chunk whose running sum crosses u * S, then its
  // elements in order (four 256-element slices, one wave scan each).
  const double thr = (double)a.u_draft[(long long)b * kDrafts + row] * S;
  auto r = [&](int c) {
    return sref[c] == -INFINITY ? 0.0 : ssum[c] * exp_from(sref[c], neg_scaled(M), a.exp_k);
  };
  double before;
  int c = block_cross(r, nsc, 0.0, thr, sh.red, sh.pick, &before);
  const RowWeights rw{x, V, vec, M, a.exp_k};
  int d = -1;
  if (c < nsc) {
    // Wave w weighs slice 4 c + w of the crossing super-chunk; the slices' sums, added in
    // slice order from `before`, name the slice that crosses, whose wave scans it.
    const int slice = c * 4 + w, v0 = slice * kWC + 4 * lane;
    double e[4] = {0.0, 0.0, 0.0, 0.0};
    if (slice * kWC < V) rw.four(v0, e);
    const double tot = wave_sum_d((e[0] + e[1]) + (e[2] + e[3]));
    if (lane == 0) sh.slice_tot[w] = tot;
    if (threadIdx.x == 0) sh.draw = -1;
    __syncthreads();
    double base = before;
    int js = -1;
    for (int j = 0; j < 4 && (c * 4 + j) * kWC < V; ++j) {
      if (base + sh.slice_tot[j] > thr) {
        js = j;
        break;
      }
      base += sh.slice_tot[j];
    }
    if (w == js) {
      const int dd = wave_scan_e(e, v0, base, thr);
      if (lane == 0) sh.draw = dd;
    }
    __syncthreads();
    d = sh.draw;
  }
  if (d < 0) {   // rounding left no crossing: the last positive weight of the row
    for (int slice = (V + kWC - 1) / kWC - 1; slice >= 0 && d < 0; --slice)
      d = wave_scan(rw, slice, 0.0, INFINITY);
  }
  if (threadIdx.x == 0) {
    if (d < 0) d = 0;
    a.draft_ids[(long long)b * kDrafts + row] = d;
    // the drawn token's draft and target logits, for the accept test
    float* pk = a.picks + ((long long)b * kDrafts + row) * 2;
    pk[0] = x[d];
    pk[1] = a.target_logits[((long long)b * kBlock + row) * V + d];
  }
}

// The request's accept decisions: one lane per draft, then the first rejection (15 if none).
__device__ int first_rejection(const SampledArgs& a, int b, const double* st) {
  const int l = threadIdx.x % kWave;
  bool reject = false;
  if (l < kDrafts) {
    const float dl = a.picks[((long long)b * kDrafts + l) * 2 + 0];
    const float tl = a.picks[((long long)b * kDrafts + l) * 2 + 1];
    const double qd = exp_from(dl, neg_scaled((float)st[2 * l]), a.exp_k) / st[2 * l + 1];
    const double pd = exp_from(tl, neg_scaled((float)st[2 * (kDrafts + l)]), a.exp_k) /
                      st[2 * (kDrafts + l) + 1];
    reject = !((double)a.u_accept[(long long)b * kDrafts + l] * qd < pd);
  }
  const unsigned long long rj = __ballot(reject) | (1ull << kDrafts);
  return __ffsll((long long)rj) - 1;
}

// The weights of the final draw for rejection index i: the residual max(0, p_i - q_i)
// (i < 15), or p_16 (p as exp(x - m) / sum of its row).
struct DrawRow {
  const float* tl;
  const float* dl;
  float mp, mq;
  double isp, isq;   // 1 / (sum of exp) of the target and draft rows
  int V;
  bool vec, residual;
  const double* ek;
  // The weights of four elements from their target (t) and draft (d) logits.
  __device__ void weights(const f32x4& t, const f32x4& d, double* e) const {
    const double kp = neg_scaled(mp), kq = neg_scaled(mq);
    const double(&kk)[4] = *reinterpret_cast<const double(*)[4]>(ek);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double p = exp_from(t[j], kp, kk) * isp;
      const double q = residual ? exp_from(d[j], kq, kk) * isq : 0.0;
      e[j] = !residual ? p : (p > q ? p - q : 0.0);
    }
  }
  __device__ void four(int v0, double* e) const {
    const f32x4 t = load4(tl, v0, V, vec);
    const f32x4 d = residual ? load4(dl, v0, V, vec) : t;
    weights(t, d, e);
  }
};

__device__ DrawRow draw_row(const SampledArgs& a, int b, int i, const double* st) {
  const int V = a.vocab;
  DrawRow r;
  r.tl = a.target_logits + ((long long)b * kBlock + i) * V;
  r.mp = (float)st[2 * (kDrafts + i)];
  r.isp = 1.0 / st[2 * (kDrafts + i) + 1];
  r.V = V;
  r.vec = (V & 3) == 0;
  r.residual = i < kDrafts;
  r.dl = r.residual ? a.draft_logits + ((long long)b * kDrafts + i) * V : r.tl;
  r.mq = r.residual ? (float)st[2 * i] : r.mp;
  r.isq = r.residual ? 1.0 / st[2 * i + 1] : r.isp;
  r.ek = a.exp_k;
  return r;
}

// Kernel 2: the chunk sums of the final draw's weights, kSegWG workgroups per request.  A
// wave takes wave chunks w, w + kSegWG * kWaves, ... and issues the loads of up to kSegBatch
// of them before the first weight.
constexpr int kSegBatch = 4;
__global__ __launch_bounds__(kThr) void sampled_segment_kernel(SampledArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int V = a.vocab, nwc = (V + kWC - 1) / kWC;
  const double* st = a.stats + (long long)b * kRows * 2;
  const int i = first_rejection(a, b, st);
  const DrawRow dw = draw_row(a, b, i, st);
  const int nfull = dw.vec ? V / kWC : 0;   // wave chunks read without bounds checks
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  constexpr int kStride = kSegWG * kWaves;
  for (int c0 = g * kWaves + w; c0 < nwc; c0 += kSegBatch * kStride) {
    f32x4 t[kSegBatch], d[kSegBatch];
#pragma unroll
    for (int u = 0; u < kSegBatch; ++u) {
      const int c = c0 + u * kStride, v0 = c * kWC + 4 * lane;
      if (c < nfull) {
        t[u] = *reinterpret_cast<const f32x4*>(dw.tl + v0);
        d[u] = dw.residual ? *reinterpret_cast<const f32x4*>(dw.dl + v0) : t[u];
      } else if (c < nwc) {
        t[u] = load4(dw.tl, v0, V, dw.vec);
        d[u] = dw.residual ? load4(dw.dl, v0, V, dw.vec) : t[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kSegBatch; ++u) {
      const int c = c0 + u * kStride;
      if (c >= nwc) break;
      double e[4];
      dw.weights(t[u], d[u], e);
      const double cs = wave_sum_d((e[0] + e[1]) + (e[2] + e[3]));
      if (lane == 0) a.chunk_sums[(long long)b * a.chunks_ld + c] = cs;
    }
  }
}

// Kernel 3: the final draw from the chunk sums, one workgroup per request.
__global__ __launch_bounds__(kThr) void sampled_draw_kernel(SampledArgs a) {
  __shared__ double red[kWaves + 1];
  __shared__ int pick[kWaves];
  extern __shared__ double psum[];   // nwc doubles: the chunk sums (then p's, below)
  const int b = blockIdx.x;
  const int V = a.vocab, nwc = (V + kWC - 1) / kWC;
  const double* st = a.stats + (long long)b * kRows * 2;
  const double* cs_g = a.chunk_sums + (long long)b * a.chunks_ld;
  for (int k = threadIdx.x; k < nwc; k += kThr) psum[k] = cs_g[k];   // the chunk sums
  const int i = first_rejection(a, b, st);
  DrawRow dw = draw_row(a, b, i, st);
  const double u = (double)a.u_resample[b];
  __syncthreads();
  const double* cs = psum;
  auto chunk = [&](int k) { return cs[k]; };
  double total;   // the chunk sums in a fixed order (no crossing at +inf)
  block_cross(chunk, nwc, 0.0, INFINITY, red, pick, &total);
  int x;
  if (total > 0.0) {
    double before;
    int c = block_cross(chunk, nwc, 0.0, u * total, red, pick, &before);
    if (c < nwc) {
      x = wave_scan(dw, c, before, u * total);
    } else {   // rounding left no crossing: the last positive weight of the row
      c = nwc - 1;
      while (c > 0 && !(cs[c] > 0.0)) --c;
      x = wave_scan(dw, c, 0.0, INFINITY);
    }
  } else {
    // No residual mass left (possible only by rounding): draw from p_i, whose chunk sums
    // are formed here, in place of the residual's.
    dw.residual = false;
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    for (int c = w; c < nwc; c += kWaves) {
      double e[4];
      dw.four(c * kWC + 4 * lane, e);
      const double s = wave_sum_d((e[0] + e[1]) + (e[2] + e[3]));
      if (lane == 0) psum[c] = s;
    }
    __syncthreads();
    auto pc = [&](int k) { return psum[k]; };
    double tp, before;
    block_cross(pc, nwc, 0.0, INFINITY, red, pick, &tp);
    int c = block_cross(pc, nwc, 0.0, u * tp, red, pick, &before);
    if (c >= nwc) c = nwc - 1;
    x = wave_scan(dw, c, before, u * tp);
  }
  const int t = threadIdx.x;
  if (t < kBlock) {
    int e = -1;
    if (t < i) e = a.draft_ids[(long long)b * kDrafts + t];
    else if (t == i) e = x < 0 ? 0 : x;
    a.emitted[(long long)b * kBlock + t] = e;
  }
  if (t == 0) a.accept_len[b] = i + 1;
}

hipError_t launch_verify_sampled(const SampledArgs& args, int batch, hipStream_t stream) {
  if (args.vocab <= 0 || args.vocab > kMaxSampledVocab) return hipErrorInvalidValue;
  SampledArgs a = args;
  a.exp_k[0] = kLog2eD;
  a.exp_k[1] = 0.69314718055994530942;    // (ln 2)^k / k!, k = 1, 2, 3
  a.exp_k[2] = 0.24022650695910071233;
  a.exp_k[3] = 0.055504108664821579953;
  const int nwc = (a.vocab + kWC - 1) / kWC, nsc = (a.vocab + kSC - 1) / kSC;
  sampled_stats_kernel<<<dim3(kRows, batch), kThr, stats_lds_bytes(nsc), stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sampled_segment_kernel<<<dim3(kSegWG, batch), kThr, 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sampled_draw_kernel<<<batch, kThr, (size_t)nwc * 8, stream>>>(a);
  return hipGetLastError();
}

size_t verify_sampled_stats_bytes(int batch, int vocab) {
  const size_t nwc = (size_t)(vocab + kWC - 1) / kWC;
  return (size_t)batch * (kRows * 2 + nwc) * sizeof(double) +
         (size_t)batch * kDrafts * 2 * sizeof(float);
}

}  // namespace dflash
