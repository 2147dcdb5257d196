// Device-side helpers shared by the DFlash kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 16;      // block slots of the temperature-1 verify: anchor + 15 masks
constexpr int kDrafts = 15;
constexpr int kPage = 16;
constexpr int kQRows = 16;      // query rows of one attention tile (one MFMA row block)
constexpr int kMaxBlock = 32;   // largest draft block (block sizes 8, 16 and 32)

// Rows of a draft pass: `rpr` rows per request (16, or 32 for a 32-token block), of which
// slots 0 .. nb-1 are the block [anchor, mask x (nb - 1)] (a block of 8 pads its request to
// 16 rows).  Slot j in 1 .. nb-1 of request b yields draft row b * (nb - 1) + j - 1; other
// rows yield none (-1).
__host__ __device__ inline long long draft_out_row(int m, int rpr, int nb) {
  const int b = m / rpr, j = m % rpr;
  return (j >= 1 && j < nb) ? (long long)b * (nb - 1) + j - 1 : -1;
}

// ---------------------------------------------------------------------------------------
// Element types.  A "k-tile" is the K extent one lane loads as 16 bytes per MFMA row/col:
// 8 bf16 or 4 fp32 per lane, 4 lane groups -> 32 (bf16) or 16 (fp32) K values per tile.
// ---------------------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<bf16> {
  static constexpr int kPerLane = 8;
  static constexpr int kTile = 32;
  __device__ static inline float to_f(bf16 v) { return (float)v; }
  __device__ static inline bf16 from_f(float v) { return (bf16)v; }
};
template <> struct Elem<float> {
  static constexpr int kPerLane = 4;
  static constexpr int kTile = 16;
  __device__ static inline float to_f(float v) { return v; }
  __device__ static inline float from_f(float v) { return v; }
};

// 16x16 output tile += A(16 x kTile) * B(kTile x 16) for one k-tile.  `a` and `b` are the
// 16-byte lane fragments: lane l holds row (A) / column (B) l % 16 and k-slice l / 16.
// Output layout: lane l holds rows 4*(l/16)+j, column l%16, j = 0..3.
template <typename T> __device__ inline f32x4 mfma_tile(i32x4 a, i32x4 b, f32x4 c);

template <> __device__ inline f32x4 mfma_tile<bf16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ inline f32x4 mfma_tile<float>(i32x4 a, i32x4 b, f32x4 c) {
  // Element-wise reinterpretation through scalars: bit-casting an ext-vector element
  // lvalue directly makes clang read element 0 for every step.
  const int a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  const int b0 = b[0], b1 = b[1], b2 = b[2], b3 = b[3];
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a0), __int_as_float(b0), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a1), __int_as_float(b1), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a2), __int_as_float(b2), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a3), __int_as_float(b3), c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------------------
// Pairs of floats to bf16 with one packed round-to-nearest-even convert (v_cvt_pk_bf16_f32).
// bf16_pair_split also leaves in a and b what the bf16 pieces did not carry (exact in
// fp32), so repeated calls peel off successive pieces.
// ---------------------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline int bf16_pair(float a, float b) {
  return __builtin_bit_cast(int, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ inline int bf16_pair_split(float& a, float& b) {
  const int hp = bf16_pair(a, b);
  a -= __int_as_float(hp << 16);
  b -= __int_as_float(hp & (int)0xffff0000u);
  return hp;
}

// ---------------------------------------------------------------------------------------
// Activation (A operand) fragments.  Activations live in memory as fp32 (or as the bf16
// target features).  For bf16 weights an fp32 activation is fed to the bf16 MFMA as a sum
// of bf16 pieces, one MFMA per piece (bf16 x bf16 products are exact in fp32).
// ---------------------------------------------------------------------------------------
template <typename WT, typename AT, int Terms = 2> struct AFrag;

template <int Terms> struct AFrag<bf16, bf16, Terms> {   // bf16 input features: exact
  static constexpr int kTerms = 1;
  i32x4 part[1];
  __device__ inline void load(const bf16* p, bool valid) {
    part[0] = valid ? *reinterpret_cast<const i32x4*>(p) : i32x4{0, 0, 0, 0};
  }
};

// fp32 activations split into Terms bf16 pieces: a = p0 + p1 (+ p2), each piece the bf16
// rounding of what the previous ones left over (the leftovers are exact in fp32).  Two
// pieces carry ~16 significant bits (relative error < 2^-16), three carry all 24.
template <int Terms> struct AFrag<bf16, float, Terms> {
  static constexpr int kTerms = Terms;
  i32x4 part[Terms];
  __device__ inline void from_floats(const float* src) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = src[i];
#pragma unroll
    for (int t = 0; t < Terms; ++t) {
      int h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = bf16_pair_split(f[2 * i], f[2 * i + 1]);
      part[t] = i32x4{h[0], h[1], h[2], h[3]};
    }
  }
};

template <int Terms> struct AFrag<float, float, Terms> {  // fp32 model
  static constexpr int kTerms = 1;
  i32x4 part[1];
  __device__ inline void from_floats(const float* f) {
    part[0] = i32x4{__float_as_int(f[0]), __float_as_int(f[1]), __float_as_int(f[2]),
                    __float_as_int(f[3])};
  }
};

// ---------------------------------------------------------------------------------------
// Wave reductions (wave64) through ds_swizzle-free shuffles.
// ---------------------------------------------------------------------------------------
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Orderable key for (value, index) argmax: larger value wins, then lower index.
__device__ inline unsigned long long argmax_key(float v, int idx) {
  unsigned u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)idx);
}
__device__ inline int argmax_key_index(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (unsigned)(k & 0xFFFFFFFFull));
}
// The value a key was made from (inverse of the order-preserving bit transform).
__device__ inline float argmax_key_value(unsigned long long k) {
  const unsigned u = (unsigned)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
// Best two keys (k1 > k2; key 0 = none): insert one key, or merge another best-two pair.
// Keys are distinct (they carry the column index), so the merge is symmetric.  Written
// with selects: the branchy form made the compiler keep these 64-bit values on the stack.
__device__ inline void top2_push(unsigned long long& k1, unsigned long long& k2,
                                 unsigned long long k) {
  const bool gt = k > k1;
  k2 = gt ? k1 : (k > k2 ? k : k2);
  k1 = gt ? k : k1;
}
__device__ inline void top2_merge(unsigned long long& k1, unsigned long long& k2,
                                  unsigned long long o1, unsigned long long o2) {
  const bool gt = o1 > k1;
  const unsigned long long n2 = gt ? (o2 > k1 ? o2 : k1) : (o1 > k2 ? o1 : k2);
  k1 = gt ? o1 : k1;
  k2 = n2;
}
// Best three keys (k1 > k2 > k3; key 0 = none).
__device__ inline void top3_push(unsigned long long& k1, unsigned long long& k2,
                                 unsigned long long& k3, unsigned long long k) {
  const bool g1 = k > k1, g2 = k > k2, g3 = k > k3;
  k3 = g2 ? k2 : (g3 ? k : k3);
  k2 = g1 ? k1 : (g2 ? k : k2);
  k1 = g1 ? k : k1;
}

// ---------------------------------------------------------------------------------------
// Fragment ("swizzled") layout of fp32 activations.  An activation matrix [M][K] that feeds
// a GEMM is stored as the GEMM's A fragments: for each 16-row m-tile and each k-tile of
// kTile = 4 * kPer columns, the 16 x kTile values are kPer / 4 blocks of 64 lanes x 4
// floats, lane l holding row l % 16 and columns kPer * (l / 16) + 4 * block + e.  Loading
// one k-tile of A is then kPer / 4 fully coalesced 1 KB reads.  Rows are padded to 16.
// Offset in floats of element (r, k) for a matrix of KT k-tiles:
// ---------------------------------------------------------------------------------------
__device__ inline long long swz_off(int r, int k, int KT, int kPer) {
  const int kTile = 4 * kPer;
  const int kt = k / kTile, kk = k % kTile;
  const int lane = (r & 15) + 16 * (kk / kPer), j = kk % kPer;
  return (((long long)(r >> 4) * KT + kt) * (kPer / 4) + j / 4) * 256 + lane * 4 + (j & 3);
}

// ---------------------------------------------------------------------------------------
// Pair fragment layout of the fp32 activations of a bf16 model.  Every such activation
// enters the bf16 MFMA as two pieces, hi = bf16(v) and lo = bf16(v - hi), so the producer
// stores the pieces ready-made: for each 16-row m-tile and 32-column k-tile, 1024 bf16 --
// the 64 lanes' hi fragments (lane l: row l % 16, columns 8 (l / 16) .. + 8), then their lo
// fragments.  Same bytes as fp32; a consumer loads each piece with one 16-byte read per lane
// and splits nothing.  Offset in bf16 elements of the hi piece of (r, k) for a matrix of KT
// k-tiles; the lo piece is kHiLoStride further.
// ---------------------------------------------------------------------------------------
constexpr int kHiLoStride = 512;
__device__ inline long long hilo_off(int r, int k, int KT) {
  const int kk = k & 31;
  const int lane = (r & 15) + 16 * (kk >> 3);
  return ((long long)(r >> 4) * KT + (k >> 5)) * 1024 + lane * 8 + (kk & 7);
}
// Store v as its hi and lo pieces at hilo offset `off`.
__device__ inline void store_hilo(bf16* base, long long off, float v) {
  const bf16 h = (bf16)v;
  base[off] = h;
  base[off + kHiLoStride] = (bf16)(v - (float)h);
}
// Store four consecutive columns k .. k + 3 (k % 4 == 0) of one row: two 8-byte stores.
__device__ inline void store_hilo4(bf16* base, long long off, f32x4 v) {
  float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
  const int h01 = bf16_pair_split(a0, a1), h23 = bf16_pair_split(a2, a3);
  *reinterpret_cast<i32x2*>(base + off) = i32x2{h01, h23};
  *reinterpret_cast<i32x2*>(base + off + kHiLoStride) = i32x2{bf16_pair(a0, a1), bf16_pair(a2, a3)};
}

// RoPE rotation for frequency `inv` (theta^(-2i/d), computed in fp64 on the host) at
// position pos: the angle pos * inv is formed and reduced modulo 2*pi in fp64 (two-part
// constant), so the fp32 sine and cosine of the reduced angle are accurate to about one fp32
// ulp for every position a cache can hold.
__device__ inline void rope_cos_sin(int pos, double inv, float* c, float* s) {
  constexpr double kTwoPiHi = 6.283185307179586;            // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;       // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double a = (double)pos * inv;
  const double k = rint(a * kInvTwoPi);
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
  sincosf((float)r, s, c);
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace dflash
