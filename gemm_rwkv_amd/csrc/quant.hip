// Round-to-nearest quantizers: weights (fp32) into the librq formats and
// per-token activations (fp16) into fp8 / int8 codes.
//
// Every scale and code is decided by IEEE fp64 operations followed by one
// round-to-nearest-even step (device_common.h), so the results are exactly
// those of the format definitions:
//   symmetric groups  s = fp16(absmax / Q), q = clamp(RNE(w / s), -Q, Q)
//     (model card "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang", Format &
//     loading: group-wise symmetric int4; Q = 127 for int8, 7 for int4)
//   asymmetric superblocks of 256 = 8 x 32 with 6-bit sub-codes
//     (rwkv-quant news article, "Dois presets e seis tamanhos")
//   per-row fp8 e4m3fn / int8 with an fp32 scale
//     (RWKV-7 Quantization Toolkit, Key Design: FP8 and INT8 GEMMs)
// No fused multiply-add may merge these steps, so contraction is off here.
#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace rq {

// Four 4-bit values of consecutive k (k % 8 == 0 for the even lane of a pair,
// 4 for the odd lane) -> the whole 32-bit code word of those 8 k, assembled
// with the partner lane: in a word even k fill the low half-word and odd k the
// high half-word, nibble i of each half holding pair i (k = 2i, 2i + 1).
// Called by both lanes of every pair (it shuffles); only the even lane stores.
__device__ __forceinline__ uint32_t nibble_word_part(uint32_t u0, uint32_t u1, uint32_t u2,
                                                     uint32_t u3, int odd) {
  const uint32_t lo = u0 | (u2 << 4), hi = u1 | (u3 << 4);  // pairs 0,1 or 2,3
  const uint32_t mine = odd ? ((lo << 8) | (hi << 24)) : (lo | (hi << 16));
  return mine | (uint32_t)__shfl_xor((int)mine, 1);
}

// flags[0] <- 1 on a non-finite input, flags[1] <- 1 on a scale overflow
// (flags may be null: per-token activation quantization reports nothing).
__device__ __forceinline__ void raise_flag(int* flags, int which) {
  if (flags) flags[which] = 1;
}

// ---------------------------------------------------------------------------
// activation-weighted (AW) scale search (rwkv-quant news article, "Dois
// presets e seis tamanhos": each group's scale and offset are chosen by a
// search weighted by E[x^2] of the input channel).  The article gives no grid:
// here 16 steps shrink the RTN scale (or both ends of a superblock group's
// range) by the factor 1 - t/32, each scored by sum_k a_k (w_k - w_hat_k)^2,
// and the smallest t within (1 + 2^-40) of the lowest score is chosen (a
// choice that does not depend on the order the score is summed in).  Step 0
// is RTN.
// ---------------------------------------------------------------------------
constexpr int kAwSteps = 16;

__device__ __forceinline__ int aw_choose(const double (&err)[kAwSteps]) {
  double emin = err[0];
#pragma unroll
  for (int t = 1; t < kAwSteps; ++t) emin = err[t] < emin ? err[t] : emin;
  const double thr = emin * (1.0 + 0x1p-40);
  int pick = kAwSteps - 1;
#pragma unroll
  for (int t = kAwSteps - 1; t >= 0; --t)
    if (err[t] <= thr) pick = t;
  return pick;
}

// importances of a lane's four channels; flags a NaN, Inf or negative one
__device__ __forceinline__ float4 aw_importance(const float* imp, int64_t k, bool active, int* flags) {
  const float4 a = active ? *(const float4*)(imp + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  const bool ok = finite_f32(a.x) && finite_f32(a.y) && finite_f32(a.z) && finite_f32(a.w) && a.x >= 0.f &&
                  a.y >= 0.f && a.z >= 0.f && a.w >= 0.f;
  if (!ok) raise_flag(flags, 0);
  return a;
}

// ---------------------------------------------------------------------------
// symmetric group RTN: one lane per 4 consecutive weights, G/4 lanes a group
// (AW: the scale comes from the search above; imp is fp32 [K])
// ---------------------------------------------------------------------------
// 5 and 6 bits: the low nibble of u = q + 2^(BITS-1) goes to the int4 layout
// and u >> 4 to the high plane.  A lane holds k = 4t .. 4t+3, half of an 8-k
// word: the even lane of a pair k = 8w + 0..3 (pairs i = 0, 1), the odd lane
// 8w + 4..7 (i = 2, 3).  6-bit: nibble i = hi(8w+2i) | hi(8w+2i+1) << 2 of a
// uint16; 5-bit: bit i = hi(8w+2i), bit 4+i = hi(8w+2i+1) of a byte.
template <int BITS>
__device__ __forceinline__ uint32_t hi_word_part(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3, int odd) {
  uint32_t mine;
  if (BITS == 6) {
    const uint32_t lo8 = (h0 | (h1 << 2)) | ((h2 | (h3 << 2)) << 4);  // pairs 0,1 (or 2,3)
    mine = odd ? (lo8 << 8) : lo8;
  } else {
    const uint32_t sh = odd ? 2u : 0u;
    mine = ((h0 | (h2 << 1)) << sh) | ((h1 | (h3 << 1)) << (4 + sh));
  }
  return mine | (uint32_t)__shfl_xor((int)mine, 1);
}

template <int BITS, int G, bool AW>
__global__ void __launch_bounds__(256) quant_sym_kernel(const float4* __restrict__ w, int64_t total4,
                                                        void* __restrict__ codes,
                                                        uint16_t* __restrict__ scales, void* __restrict__ hi,
                                                        int* __restrict__ flags, const float* __restrict__ imp,
                                                        int64_t K) {
  constexpr int LPG = G / 4;
  constexpr int Q = (1 << (BITS - 1)) - 1;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool active = t < total4;
  float4 v = active ? w[t] : make_float4(0.f, 0.f, 0.f, 0.f);
  const bool fin = finite_f32(v.x) && finite_f32(v.y) && finite_f32(v.z) && finite_f32(v.w);
  if (!fin) raise_flag(flags, 0);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = group_max<LPG>(a);
  uint16_t sbits;
  if constexpr (AW) {
    const float4 av = aw_importance(imp, (t * 4) % K, active, flags);
    const float e4[4] = {v.x, v.y, v.z, v.w}, a4[4] = {av.x, av.y, av.z, av.w};
    const double base = (double)a / (double)Q;
    if (f64_to_f16_bits(base) == 0x7c00u) raise_flag(flags, 1);  // step 0 overflows iff any step does
    double err[kAwSteps];
#pragma unroll
    for (int st = 0; st < kAwSteps; ++st) {
      const double s = f16_bits_to_f64(f64_to_f16_bits(base * (1.0 - st / 32.0)));
      double e = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double r = s == 0.0 ? 0.0 : __builtin_rint((double)e4[i] / s);
        r = r > (double)Q ? (double)Q : (r < -(double)Q ? -(double)Q : r);
        const double d = (double)e4[i] - r * s;
        e = e + (double)a4[i] * (d * d);
      }
      err[st] = group_sum_d<LPG>(e);
    }
    sbits = f64_to_f16_bits(base * (1.0 - aw_choose(err) / 32.0));
  } else {
    sbits = f64_to_f16_bits((double)a / (double)Q);
  }
  if (sbits == 0x7c00u) raise_flag(flags, 1);
  const double s = f16_bits_to_f64(sbits);
  int q[4];
  const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double r = s == 0.0 ? 0.0 : __builtin_rint((double)e[i] / s);
    r = r > (double)Q ? (double)Q : (r < -(double)Q ? -(double)Q : r);
    q[i] = (int)r;
  }
  if (BITS == 8) {
    uint32_t packed = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                      ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
    if (active) ((uint32_t*)codes)[t] = packed;
  } else {
    constexpr int OFF = 1 << (BITS - 1);
    const uint32_t u0 = (uint32_t)(q[0] + OFF), u1 = (uint32_t)(q[1] + OFF), u2 = (uint32_t)(q[2] + OFF),
                   u3 = (uint32_t)(q[3] + OFF);
    const uint32_t w = nibble_word_part(u0 & 15u, u1 & 15u, u2 & 15u, u3 & 15u, t & 1);
    if (active && (t & 1) == 0) ((uint32_t*)codes)[t >> 1] = w;
    if constexpr (BITS == 5 || BITS == 6) {
      // lane t holds k = 4t .. 4t+3: pairs (k, k+1) = (u0, u1) and (u2, u3)
      const uint32_t h = hi_word_part<BITS>(u0 >> 4, u1 >> 4, u2 >> 4, u3 >> 4, t & 1);
      if (active && (t & 1) == 0) {
        if (BITS == 6) ((uint16_t*)hi)[t >> 1] = (uint16_t)h;
        else ((uint8_t*)hi)[t >> 1] = (uint8_t)h;
      }
    }
  }
  if (active && (t % LPG) == 0) scales[t / LPG] = sbits;
}

// ---------------------------------------------------------------------------
// asymmetric 4-bit superblocks: one wave per 256 weights, 8 lanes per group
// ---------------------------------------------------------------------------
template <bool AW>
__global__ void __launch_bounds__(256) quant_sb256_kernel(const float4* __restrict__ w, int64_t nsb,
                                                          uint32_t* __restrict__ qs,
                                                          uint16_t* __restrict__ dout,
                                                          uint16_t* __restrict__ mout,
                                                          uint32_t* __restrict__ sub,
                                                          int* __restrict__ flags, const float* __restrict__ imp,
                                                          int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t sbi = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (sbi >= nsb) return;  // uniform per wave
  const float4 v = w[sbi * 64 + lane];
  const bool fin = finite_f32(v.x) && finite_f32(v.y) && finite_f32(v.z) && finite_f32(v.w);
  if (!fin) raise_flag(flags, 0);
  float hi = group_max<8>(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  float lo = fminf(0.f, group_min<8>(fminf(fminf(v.x, v.y), fminf(v.z, v.w))));
  double s, nl;
  if constexpr (AW) {
    // the group's range ends scaled toward zero, scored with the unquantized
    // scale s_t and offset m_t; the chosen pair goes through the superblock step
    const float4 av = aw_importance(imp, (sbi * 256 + lane * 4) % K, true, flags);
    const float e4[4] = {v.x, v.y, v.z, v.w}, a4[4] = {av.x, av.y, av.z, av.w};
    double err[kAwSteps];
#pragma unroll
    for (int st = 0; st < kAwSteps; ++st) {
      const double f = 1.0 - st / 32.0;
      const double lo_t = (double)lo * f, hi_t = (double)hi * f;
      double sv = (hi_t - lo_t) / 15.0;
      if (sv == 0.0) sv = 0.0;
      const double mv = 0.0 - lo_t;
      double e = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double u = sv == 0.0 ? 0.0 : __builtin_rint(((double)e4[i] + mv) / sv);
        u = u < 0.0 ? 0.0 : (u > 15.0 ? 15.0 : u);
        const double d = (double)e4[i] - (sv * u - mv);
        e = e + (double)a4[i] * (d * d);
      }
      err[st] = group_sum_d<8>(e);
    }
    const double f = 1.0 - aw_choose(err) / 32.0;
    const double lo_t = (double)lo * f, hi_t = (double)hi * f;
    s = (hi_t - lo_t) / 15.0;
    if (s == 0.0) s = 0.0;
    nl = 0.0 - lo_t;
  } else {
    s = ((double)hi - (double)lo) / 15.0;
    if (s == 0.0) s = 0.0;  // a zero range is +0
    nl = 0.0 - (double)lo;
  }
  const double smax = group_max_d<64>(s);
  const double nlmax = group_max_d<64>(nl);
  const uint16_t db = f64_to_f16_bits(smax / 63.0);
  const uint16_t mb = f64_to_f16_bits(nlmax / 63.0);
  if (db == 0x7c00u || mb == 0x7c00u) raise_flag(flags, 1);
  const double dd = f16_bits_to_f64(db);
  const double dm = f16_bits_to_f64(mb);
  double sc = dd == 0.0 ? 0.0 : __builtin_rint(s / dd);
  double mc = dm == 0.0 ? 0.0 : __builtin_rint(nl / dm);
  sc = sc < 0.0 ? 0.0 : (sc > 63.0 ? 63.0 : sc);
  mc = mc < 0.0 ? 0.0 : (mc > 63.0 ? 63.0 : mc);
  const double S = dd * sc;
  const double M = dm * mc;
  const float e[4] = {v.x, v.y, v.z, v.w};
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double r = S == 0.0 ? 0.0 : __builtin_rint(((double)e[i] + M) / S);
    r = r < 0.0 ? 0.0 : (r > 15.0 ? 15.0 : r);
    u[i] = (uint32_t)r;
  }
  const uint32_t qw = nibble_word_part(u[0], u[1], u[2], u[3], lane & 1);
  if ((lane & 1) == 0) qs[sbi * 32 + (lane >> 1)] = qw;
  // gather the eight 6-bit pairs into lane 0
  const uint32_t isc = (uint32_t)sc, imc = (uint32_t)mc;
  uint64_t lo48 = 0, hi48 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo48 |= (uint64_t)__shfl(isc, 8 * j) << (6 * j);
    hi48 |= (uint64_t)__shfl(imc, 8 * j) << (6 * j);
  }
  if (lane == 0) {
    dout[sbi] = db;
    mout[sbi] = mb;
    uint32_t* o = sub + sbi * 3;
    o[0] = (uint32_t)lo48;
    o[1] = (uint32_t)(lo48 >> 32) | ((uint32_t)hi48 << 16);
    o[2] = (uint32_t)(hi48 >> 16);
  }
}

// ---------------------------------------------------------------------------
// per-row fp8 / int8: one workgroup per row, scale from the row's absmax
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&o)[4]);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&o)[4]) {
  float4 v = *(const float4*)p;
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}

template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float (&o)[4]) {
  uint2 v = *(const uint2*)p;
  o[0] = f16_bits_to_f32((uint16_t)(v.x & 0xffff));
  o[1] = f16_bits_to_f32((uint16_t)(v.x >> 16));
  o[2] = f16_bits_to_f32((uint16_t)(v.y & 0xffff));
  o[3] = f16_bits_to_f32((uint16_t)(v.y >> 16));
}

// One code against the stored per-row scale s (a decoded fp32, here in fp64):
// the fp64 quotient rounded onto the fp8 e4m3fn grid (saturating) or to a
// clamped int8.  A zero scale gives code 0.
template <bool FP8>
__device__ __forceinline__ uint32_t row_code(float e, double s) {
  if (s == 0.0) return 0u;
  if (FP8) return f64_to_e4m3((double)e / s);
  double q = __builtin_rint((double)e / s);
  q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
  return (uint32_t)((int)q & 0xff);
}

template <typename T, bool FP8>
__global__ void __launch_bounds__(256) quant_rows_kernel(const T* __restrict__ in, int64_t k, int64_t ld,
                                                         uint32_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         int* __restrict__ flags) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* r = in + row * ld;
  const int64_t k4 = k >> 2;
  float a = 0.f;
  bool fin = true;
  for (int64_t i = threadIdx.x; i < k4; i += 256) {
    float e[4];
    load4<T>(r + 4 * i, e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fin = fin && finite_f32(e[j]);
      a = fmaxf(a, fabsf(e[j]));
    }
  }
  if (!fin) raise_flag(flags, 0);
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const uint32_t sb = f64_to_f32_bits((double)a / (FP8 ? 448.0 : 127.0));
  if (sb == 0x7f800000u) raise_flag(flags, 1);
  const double s = (double)__builtin_bit_cast(float, sb);
  uint32_t* out = codes + row * k4;
  for (int64_t i = threadIdx.x; i < k4; i += 256) {
    float e[4];
    load4<T>(r + 4 * i, e);
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) packed |= row_code<FP8>(e[j], s) << (8 * j);
    out[i] = packed;
  }
  if (threadIdx.x == 0) scales[row] = __builtin_bit_cast(float, sb);
}

// Per-token quantization of fp16 activations in one pass: a workgroup per
// row, each thread loads its NL blocks of 8 halves at once and keeps them in
// registers through the row's absmax reduction and the coding.  Same codes
// and scales as quant_rows_kernel; rows of up to 2048 blocks (K <= 16384).
template <bool FP8, int NL>
__global__ void __launch_bounds__(1024) quant_act_kernel(const uint16_t* __restrict__ x, int k, int64_t ldx,
                                                         uint2* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         int* __restrict__ flags) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const uint16_t* r = x + row * ldx;
  const int blocks = k >> 3;
  uint4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int b = threadIdx.x + i * blockDim.x;
    v[i] = b < blocks ? *(const uint4*)(r + 8 * b) : make_uint4(0u, 0u, 0u, 0u);
  }
  float a = 0.f;
  bool fin = true;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = f16_bits_to_f32((uint16_t)(w[j >> 1] >> (16 * (j & 1))));
      fin = fin && finite_f32(e);
      a = fmaxf(a, fabsf(e));
    }
  }
  if (!fin) raise_flag(flags, 0);
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) a = fmaxf(a, red[w]);
  const uint32_t sb = f64_to_f32_bits((double)a / (FP8 ? 448.0 : 127.0));
  if (sb == 0x7f800000u) raise_flag(flags, 1);
  const double s = (double)__builtin_bit_cast(float, sb);
  uint2* out = codes + row * blocks;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int b = threadIdx.x + i * blockDim.x;
    if (b >= blocks) continue;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= row_code<FP8>(f16_bits_to_f32((uint16_t)(w[j >> 1] >> (16 * (j & 1)))), s) << (8 * j);
      hi |= row_code<FP8>(f16_bits_to_f32((uint16_t)(w[2 + (j >> 1)] >> (16 * (j & 1)))), s) << (8 * j);
    }
    out[b] = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scales[row] = __builtin_bit_cast(float, sb);
}

// ---------------------------------------------------------------------------
// fp32 -> fp16 (RNE) for unquantized head weights
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) to_f16_kernel(const float* __restrict__ w, int64_t count,
                                                     uint16_t* __restrict__ out, int* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float v = w[i];
  if (!finite_f32(v)) raise_flag(flags, 0);
  const uint16_t h = f64_to_f16_bits((double)v);
  if ((h & 0x7fffu) == 0x7c00u) raise_flag(flags, 1);
  out[i] = h;
}

// fp32 -> bfloat16, round to nearest with ties to even: add 0x7fff plus the
// lowest kept bit to the fp32 pattern and keep the top half (a carry out of
// the mantissa moves the exponent up, which is the correct rounding; past
// the largest finite value it gives infinity, reported as a range error)
__global__ void __launch_bounds__(256) to_bf16_kernel(const float* __restrict__ w, int64_t count,
                                                      uint16_t* __restrict__ out, int* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float v = w[i];
  if (!finite_f32(v)) raise_flag(flags, 0);
  const uint32_t b = __float_as_uint(v);
  const uint16_t h = (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
  if ((h & 0x7fffu) == 0x7f80u) raise_flag(flags, 1);
  out[i] = h;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quant_sym(const float* w, int64_t n, int64_t k, int bits, int group, void* codes,
                            uint16_t* scales, void* hi, int* flags, const float* imp, hipStream_t st) {
  const int64_t total4 = n * k / 4;
  if (total4 == 0) return hipSuccess;
  const dim3 grid(grid_for(total4)), block(256);
  const float4* w4 = (const float4*)w;
#define RQ_SYM_CASE(B, G)                                                                          \
  if (bits == B && group == G) {                                                                   \
    if (imp)                                                                                       \
      hipLaunchKernelGGL((quant_sym_kernel<B, G, true>), grid, block, 0, st, w4, total4, codes,    \
                         scales, hi, flags, imp, k);                                               \
    else                                                                                           \
      hipLaunchKernelGGL((quant_sym_kernel<B, G, false>), grid, block, 0, st, w4, total4, codes,   \
                         scales, hi, flags, imp, k);                                               \
    return hipGetLastError();                                                                      \
  }
  RQ_SYM_CASE(8, 16)
  RQ_SYM_CASE(8, 32)
  RQ_SYM_CASE(8, 64)
  RQ_SYM_CASE(4, 16)
  RQ_SYM_CASE(4, 32)
  RQ_SYM_CASE(4, 64)
  RQ_SYM_CASE(6, 32)
  RQ_SYM_CASE(6, 64)
  RQ_SYM_CASE(5, 32)
  RQ_SYM_CASE(5, 64)
#undef RQ_SYM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_quant_sb256(const float* w, int64_t n, int64_t k, void* qs, void* d, void* dmin,
                              void* sub, int* flags, const float* imp, hipStream_t st) {
  const int64_t nsb = n * k / 256;
  if (nsb == 0) return hipSuccess;
  if (imp)
    hipLaunchKernelGGL(quant_sb256_kernel<true>, dim3(grid_for(nsb * 64)), dim3(256), 0, st, (const float4*)w,
                       nsb, (uint32_t*)qs, (uint16_t*)d, (uint16_t*)dmin, (uint32_t*)sub, flags, imp, k);
  else
    hipLaunchKernelGGL(quant_sb256_kernel<false>, dim3(grid_for(nsb * 64)), dim3(256), 0, st, (const float4*)w,
                       nsb, (uint32_t*)qs, (uint16_t*)d, (uint16_t*)dmin, (uint32_t*)sub, flags, imp, k);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f32(const float* w, int64_t n, int64_t k, bool fp8, void* codes,
                                 float* scales, int* flags, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL((quant_rows_kernel<float, true>), dim3((unsigned)n), dim3(256), 0, st, w, k, k,
                       (uint32_t*)codes, scales, flags);
  else
    hipLaunchKernelGGL((quant_rows_kernel<float, false>), dim3((unsigned)n), dim3(256), 0, st, w, k, k,
                       (uint32_t*)codes, scales, flags);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f16(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, bool fp8,
                                 void* codes, float* scales, int* flags, hipStream_t st) {
  if (m == 0) return hipSuccess;
  const int64_t blocks = k / 8;
  if (k % 8 == 0 && blocks <= 2048) {
    const unsigned threads = blocks <= 256 ? 256u : (blocks <= 512 ? 512u : 1024u);
    const dim3 grid((unsigned)m), block(threads);
    uint2* c2 = (uint2*)codes;
    if (blocks <= 1024) {
      if (fp8)
        hipLaunchKernelGGL((quant_act_kernel<true, 1>), grid, block, 0, st, x, (int)k, ldx, c2, scales, flags);
      else
        hipLaunchKernelGGL((quant_act_kernel<false, 1>), grid, block, 0, st, x, (int)k, ldx, c2, scales, flags);
    } else {
      if (fp8)
        hipLaunchKernelGGL((quant_act_kernel<true, 2>), grid, block, 0, st, x, (int)k, ldx, c2, scales, flags);
      else
        hipLaunchKernelGGL((quant_act_kernel<false, 2>), grid, block, 0, st, x, (int)k, ldx, c2, scales, flags);
    }
    return hipGetLastError();
  }
  if (fp8)
    hipLaunchKernelGGL((quant_rows_kernel<uint16_t, true>), dim3((unsigned)m), dim3(256), 0, st, x, k,
                       ldx, (uint32_t*)codes, scales, flags);
  else
    hipLaunchKernelGGL((quant_rows_kernel<uint16_t, false>), dim3((unsigned)m), dim3(256), 0, st, x, k,
                       ldx, (uint32_t*)codes, scales, flags);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* w, int64_t count, uint16_t* out, int* flags, hipStream_t st) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_for(count)), dim3(256), 0, st, w, count, out, flags);
  return hipGetLastError();
}

hipError_t launch_to_f16(const float* w, int64_t count, uint16_t* out, int* flags, hipStream_t st) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(to_f16_kernel, dim3(grid_for(count)), dim3(256), 0, st, w, count, out, flags);
  return hipGetLastError();
}

}  // namespace rq
