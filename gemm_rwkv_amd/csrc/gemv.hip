// Weight-streaming products for decode batches 1 <= m <= 32:
//   y[m][n] = fp16( sum_g scale(n, g) * sum_{k in g} x[m][k] * q[n][k] )
// read straight from the packed codes (no dequantized copy is written:
// RWKV-7 Quantization Toolkit, Key Design; model card "RWKV-7 G1 1.5B -- int4
// GPTQ for rwkv-sglang", summary: int4 GEMV / small-M GEMM family).
//
// Design for gfx950 (wave64, MFMA):
//   * A wave owns a tile of 16 weight rows and a slice of the K groups; the
//     waves of a workgroup split K and combine their partial sums through LDS
//     in a fixed order (deterministic, no atomics).
//   * Each lane streams the codes of one row (lane % 16) for a quarter of
//     every group (lane / 16), so a group's 16 rows x group bytes arrive in one
//     load instruction per wave.
//   * Codes become exact fp16 integers in registers with one AND-OR per two
//     codes (the code lands in the mantissa of 1024 or 64, then that bias is
//     subtracted exactly), and go into v_mfma_f32_16x16x{32,16}_f16 as the B
//     operand; activations (rows >= m are zero) are the A operand.  Products
//     are exact and accumulate in fp32 inside the MFMA.
//   * Each group's MFMA result is scaled by its fp16 scale in fp32 (symmetric
//     formats), or by S_j and corrected by M_j * sum(x) (asymmetric
//     superblocks, with sum(x) from one MFMA against ones), so the effective
//     weight q*s is exact.
//   * Decoding packs codes in the order (0,4,1,5,2,6,3,7) (int4) or
//     (0,2,1,3,...) (int8); the activation fragment is permuted to match with
//     v_perm_b32, which is free to choose because a dot product does not
//     depend on the order of its terms.
#include "device_common.h"
#include "kernels.h"

namespace rq {

// ---------------------------------------------------------------------------
// per-format traits
// ---------------------------------------------------------------------------
// GK: k per scale group (32 for SB and F16, where F16 has no scale)
// LK: k per lane per group (GK / 4), LKM: k per lane per MFMA (8 or 4)
template <int FMT, int G>
struct Fmt {
  static constexpr int GK = (FMT == GF_SB || FMT == GF_F16) ? 32 : G;
  static constexpr int LK = GK / 4;
  static constexpr int LKM = LK >= 8 ? 8 : 4;
  static constexpr int NT = LK / LKM;  // MFMAs per group
  // code bytes per lane per group
  static constexpr int LB = FMT == GF_W8 ? LK : (FMT == GF_F16 ? LK * 2 : LK / 2);
  // code bytes per row per group
  static constexpr int RB = LB * 4;
};

template <int B>
struct Bytes;
template <>
struct Bytes<2> { typedef uint16_t T; };
template <>
struct Bytes<4> { typedef uint32_t T; };
template <>
struct Bytes<8> { typedef uint2 T; };
template <>
struct Bytes<16> { typedef uint4 T; };

__device__ __forceinline__ uint32_t w_at(uint16_t v, int) { return v; }
__device__ __forceinline__ uint32_t w_at(uint32_t v, int) { return v; }
__device__ __forceinline__ uint32_t w_at(uint2 v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t w_at(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t hsub2(uint32_t a, uint32_t b) {
  half2v r = __builtin_bit_cast(half2v, a) - __builtin_bit_cast(half2v, b);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 int4 codes (one word, k order 0..7) -> fp16 (q - bias) in order 0,4,1,5,2,6,3,7.
// bias_lo/bias_hi: 1032 / 72 for offset-binary symmetric codes, 1024 / 64 for
// unsigned superblock codes.
template <bool SIGNED>
__device__ __forceinline__ half8 dec_w4x8(uint32_t v) {
  const uint32_t b1024 = SIGNED ? 0x64086408u : 0x64006400u;  // 1032 : 1024
  const uint32_t b64 = SIGNED ? 0x54805480u : 0x54005400u;    // 72 : 64
  uint32_t v8 = v >> 8;
  uint32_t h0 = hsub2((v & 0x000f000fu) | 0x64006400u, b1024);
  uint32_t h1 = hsub2((v & 0x00f000f0u) | 0x54005400u, b64);
  uint32_t h2 = hsub2((v8 & 0x000f000fu) | 0x64006400u, b1024);
  uint32_t h3 = hsub2((v8 & 0x00f000f0u) | 0x54005400u, b64);
  uint4 r = make_uint4(h0, h1, h2, h3);
  return __builtin_bit_cast(half8, r);
}

// 4 int4 codes (16 bits, k order 0..3) -> fp16 in order 0,2,1,3
__device__ __forceinline__ half4 dec_w4x4(uint32_t v) {
  uint32_t t = perm(0u, v, 0x0c010c00u);  // bytes: b0, 0, b1, 0
  uint32_t h0 = hsub2((t & 0x000f000fu) | 0x64006400u, 0x64086408u);
  uint32_t h1 = hsub2((t & 0x00f000f0u) | 0x54005400u, 0x54805480u);
  uint2 r = make_uint2(h0, h1);
  return __builtin_bit_cast(half4, r);
}

// 4 int8 codes (one word, k order 0..3) -> fp16 in order 0,2,1,3
__device__ __forceinline__ uint2 dec_w8x4_raw(uint32_t v) {
  uint32_t u = v ^ 0x80808080u;                            // q + 128 in each byte
  uint32_t lo = perm(0x64646464u, u, 0x04020400u);          // (1024+u0, 1024+u2)
  uint32_t hi = perm(0x64646464u, u, 0x04030401u);          // (1024+u1, 1024+u3)
  return make_uint2(hsub2(lo, 0x64806480u), hsub2(hi, 0x64806480u));  // - 1152
}

// activation permutations matching the decoders
// natural halves d0=(x0,x1) d1=(x2,x3) d2=(x4,x5) d3=(x6,x7)
__device__ __forceinline__ half8 xperm_w4x8(uint4 d) {
  uint4 r = make_uint4(perm(d.z, d.x, 0x05040100u), perm(d.z, d.x, 0x07060302u),
                       perm(d.w, d.y, 0x05040100u), perm(d.w, d.y, 0x07060302u));
  return __builtin_bit_cast(half8, r);
}
__device__ __forceinline__ half8 xperm_w8x8(uint4 d) {
  uint4 r = make_uint4(perm(d.y, d.x, 0x05040100u), perm(d.y, d.x, 0x07060302u),
                       perm(d.w, d.z, 0x05040100u), perm(d.w, d.z, 0x07060302u));
  return __builtin_bit_cast(half8, r);
}
__device__ __forceinline__ half4 xperm_x4(uint2 d) {
  uint2 r = make_uint2(perm(d.y, d.x, 0x05040100u), perm(d.y, d.x, 0x07060302u));
  return __builtin_bit_cast(half4, r);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// MT: number of 16-row activation tiles (1: m <= 16, 2: m <= 32)
// NW: waves per workgroup, splitting the groups of K
// U : groups loaded ahead per step
template <int FMT, int G, int MT, int NW, int U>
__global__ void __launch_bounds__(NW * 64) gemv_kernel(const GemvBatch p) {
  typedef Fmt<FMT, G> F;
  typedef typename Bytes<F::LB>::T CodeT;
  constexpr int LKM = F::LKM;
  constexpr int NT = F::NT;
  constexpr int GK = F::GK;

  __shared__ float red[NW > 1 ? NW : 1][MT][4][64];

  // which matrix and row tile
  int tile = blockIdx.x;
  int mi = 0;
  if (tile >= p.mat[0].tiles) {
    tile -= p.mat[0].tiles;
    mi = 1;
    if (tile >= p.mat[1].tiles) {
      tile -= p.mat[1].tiles;
      mi = 2;
    }
  }
  const GemvMatrix& A = p.mat[mi];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;   // B column = weight row within the tile; also A row
  const int kq = lane >> 4;  // quarter of a group
  const int n = tile * 16 + j;
  const bool nvalid = n < A.n;
  const int nrow = nvalid ? n : 0;
  const int k = p.k;
  const int ng = k / GK;
  const int per = (ng + NW - 1) / NW;
  const int g0 = wave * per;
  const int g1 = min(ng, g0 + per);

  const uint8_t* crow = (const uint8_t*)A.codes + (size_t)nrow * (size_t)(ng * F::RB) + kq * F::LB;
  const uint16_t* srow = nullptr;
  const uint16_t* mrow = nullptr;
  const uint32_t* subrow = nullptr;
  if constexpr (FMT == GF_W4 || FMT == GF_W8) srow = A.scales + (size_t)nrow * ng;
  if constexpr (FMT == GF_SB) {
    srow = A.scales + (size_t)nrow * (ng / 8);
    mrow = A.mins + (size_t)nrow * (ng / 8);
    subrow = A.sub + (size_t)nrow * (ng / 8) * 3;
  }
  // activation rows held by this lane (A operand rows), zero beyond m
  bool mval[MT];
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = t * 16 + j;
    mval[t] = m < p.m;
    xrow[t] = A.x + (size_t)(mval[t] ? m : 0) * p.ldx + kq * F::LK;
  }

  float4v acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int gb = g0; gb < g1; gb += U) {
    CodeT cw[U];
    float sc[U];
    float mn[U];
    uint4 xv[U][MT][NT > 1 ? 2 : 1];
    // ---- loads
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = gb + u;
      const bool gv = g < g1;
      if (gv && nvalid) {
        cw[u] = *(const CodeT*)(crow + (size_t)g * F::RB);
      } else {
        cw[u] = CodeT{};
      }
      if constexpr (FMT == GF_W4 || FMT == GF_W8) {
        sc[u] = (gv && nvalid) ? f16_bits_to_f32(srow[g]) : 0.f;
      } else if constexpr (FMT == GF_SB) {
        const int sb = g >> 3, gj = g & 7;
        if (gv && nvalid) {
          const uint32_t* sw = subrow + sb * 3;
          const uint32_t w0 = sw[0], w1 = sw[1], w2 = sw[2];
          const uint64_t lo48 = (uint64_t)w0 | ((uint64_t)(w1 & 0xffffu) << 32);
          const uint64_t hi48 = (uint64_t)(w1 >> 16) | ((uint64_t)w2 << 16);
          const uint32_t scode = (uint32_t)(lo48 >> (6 * gj)) & 63u;
          const uint32_t mcode = (uint32_t)(hi48 >> (6 * gj)) & 63u;
          sc[u] = f16_bits_to_f32(srow[sb]) * (float)scode;  // exact: 11 x 6 bits
          mn[u] = f16_bits_to_f32(mrow[sb]) * (float)mcode;
        } else {
          sc[u] = 0.f;
          mn[u] = 0.f;
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint16_t* xp = xrow[t] + (size_t)g * GK;
        if (gv && mval[t]) {
          if constexpr (F::LK == 16) {
            xv[u][t][0] = *(const uint4*)xp;
            if constexpr (NT > 1) xv[u][t][NT > 1 ? 1 : 0] = *(const uint4*)(xp + 8);
          } else if constexpr (F::LK == 8) {
            xv[u][t][0] = *(const uint4*)xp;
          } else {
            uint2 h = *(const uint2*)xp;
            xv[u][t][0] = make_uint4(h.x, h.y, 0u, 0u);
          }
        } else {
          xv[u][t][0] = make_uint4(0u, 0u, 0u, 0u);
          if constexpr (NT > 1) xv[u][t][NT > 1 ? 1 : 0] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    // ---- math
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float4v grp[MT];
      float4v xs[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        grp[t] = float4v{0.f, 0.f, 0.f, 0.f};
        xs[t] = float4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if constexpr (LKM == 8) {
          half8 b;
          if constexpr (FMT == GF_W4) {
            b = dec_w4x8<true>(w_at(cw[u], s));
          } else if constexpr (FMT == GF_SB) {
            b = dec_w4x8<false>(w_at(cw[u], s));
          } else if constexpr (FMT == GF_W8) {
            uint2 lo = dec_w8x4_raw(w_at(cw[u], 2 * s));
            uint2 hi = dec_w8x4_raw(w_at(cw[u], 2 * s + 1));
            b = __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            b = __builtin_bit_cast(half8, cw[u]);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            half8 a;
            if constexpr (FMT == GF_W4 || FMT == GF_SB)
              a = xperm_w4x8(xv[u][t][s]);
            else if constexpr (FMT == GF_W8)
              a = xperm_w8x8(xv[u][t][s]);
            else
              a = __builtin_bit_cast(half8, xv[u][t][s]);
            if constexpr (FMT == GF_F16) {
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
            } else {
              grp[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, grp[t], 0, 0, 0);
              if constexpr (FMT == GF_SB) {
                const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
                xs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, xs[t], 0, 0, 0);
              }
            }
          }
        } else {  // 4 k per lane: 16x16x16
          half4 b;
          if constexpr (FMT == GF_W4) {
            b = dec_w4x4(w_at(cw[u], 0));
          } else {
            uint2 r = dec_w8x4_raw(w_at(cw[u], 0));
            b = __builtin_bit_cast(half4, r);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            half4 a = xperm_x4(make_uint2(xv[u][t][0].x, xv[u][t][0].y));
            grp[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, grp[t], 0, 0, 0);
          }
        }
      }
      if constexpr (FMT != GF_F16) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[t][r] += sc[u] * grp[t][r];
            if constexpr (FMT == GF_SB) acc[t][r] -= mn[u] * xs[t][r];
          }
        }
      }
    }
  }

  // ---- combine the waves' partial sums, in wave order, and store fp16
  // lane holds D[m = 16t + 4*kq + r][n = tile*16 + j]
  if constexpr (NW > 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][t][r][lane] = acc[t][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * 4 * 64; idx += NW * 64) {
      const int t = idx / 256, r = (idx / 64) & 3, l = idx & 63;
      float v = red[0][t][r][l];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[w][t][r][l];
      const int m = t * 16 + 4 * (l >> 4) + r;
      const int nn = tile * 16 + (l & 15);
      if (m < p.m && nn < A.n) A.y[(size_t)m * p.ldy + nn] = f32_to_f16_bits(v);
    }
  } else {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = t * 16 + 4 * kq + r;
        if (m < p.m && nvalid) A.y[(size_t)m * p.ldy + n] = f32_to_f16_bits(acc[t][r]);
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int FMT, int G, int MT, int NW>
static hipError_t launch_t(const GemvBatch& b, hipStream_t st) {
  constexpr int U = Fmt<FMT, G>::GK == 16 ? 8 : (Fmt<FMT, G>::GK == 32 ? 4 : 2);
  int tiles = 0;
  for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemv_kernel<FMT, G, MT, NW, U>), dim3(tiles), dim3(NW * 64), 0, st, b);
  return hipGetLastError();
}

template <int FMT, int G, int MT>
static hipError_t launch_nw(const GemvBatch& b, hipStream_t st) {
  const int gk = Fmt<FMT, G>::GK;
  const int ng = b.k / gk;
  // enough groups per wave to keep several loads in flight
  if (ng >= 8 * 16) return launch_t<FMT, G, MT, 8>(b, st);
  if (ng >= 4 * 8) return launch_t<FMT, G, MT, 4>(b, st);
  if (ng >= 2 * 4) return launch_t<FMT, G, MT, 2>(b, st);
  return launch_t<FMT, G, MT, 1>(b, st);
}

template <int FMT, int G>
static hipError_t launch_mt(const GemvBatch& b, hipStream_t st) {
  if (b.m <= 16) return launch_nw<FMT, G, 1>(b, st);
  return launch_nw<FMT, G, 2>(b, st);
}

hipError_t launch_gemv(const GemvBatch& b, int fmt, int group, hipStream_t st) {
  if (b.m == 0) return hipSuccess;
  switch (fmt) {
    case GF_W4:
      if (group == 64) return launch_mt<GF_W4, 64>(b, st);
      if (group == 32) return launch_mt<GF_W4, 32>(b, st);
      if (group == 16) return launch_mt<GF_W4, 16>(b, st);
      break;
    case GF_W8:
      if (group == 64) return launch_mt<GF_W8, 64>(b, st);
      if (group == 32) return launch_mt<GF_W8, 32>(b, st);
      if (group == 16) return launch_mt<GF_W8, 16>(b, st);
      break;
    case GF_SB:
      return launch_mt<GF_SB, 32>(b, st);
    case GF_F16:
      return launch_mt<GF_F16, 32>(b, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace rq
