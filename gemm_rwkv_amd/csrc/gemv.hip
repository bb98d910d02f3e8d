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
//   * Where a decoder yields codes out of k order ((0,2,1,3,...) for int8 in
//     this kernel, one parity of an int4 word for int4 group 16) the
//     activation fragment is permuted to match with v_perm_b32, which is free
//     to choose because a dot product does not depend on the order of its
//     terms.
#include <type_traits>

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


// One half-word of an int4 code word (4 codes of one parity: k offsets
// 0, 2, 4, 6 from the lane's first k) -> fp16 q in order 0, 4, 2, 6
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
__device__ __forceinline__ half8 xperm_w8x8(uint4 d) {
  uint4 r = make_uint4(perm(d.y, d.x, 0x05040100u), perm(d.y, d.x, 0x07060302u),
                       perm(d.w, d.z, 0x05040100u), perm(d.w, d.z, 0x07060302u));
  return __builtin_bit_cast(half8, r);
}
// x for dec_w4x4: natural halves d (8 k from the word's first k), the
// lane's parity picked by sel (0x05040100 even, 0x07060302 odd)
__device__ __forceinline__ half4 xsel_w4x4(uint4 d, uint32_t sel) {
  uint2 r = make_uint2(perm(d.z, d.x, sel), perm(d.w, d.y, sel));
  return __builtin_bit_cast(half4, r);
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
  constexpr bool W4Q = FMT == GF_W4 && F::LK == 4;
  bool mval[MT];
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = t * 16 + j;
    mval[t] = m < p.m;
    // int4 with 4 k per lane: the lane's codes are one parity of the code
    // word at k 8 * (kq / 2); its x come from the 8 k of that word
    xrow[t] = A.x + (size_t)(mval[t] ? m : 0) * p.ldx + (W4Q ? 8 * (kq >> 1) : kq * F::LK);
  }
  const uint32_t xsel = (kq & 1) ? 0x07060302u : 0x05040100u;
  (void)xsel;

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
          } else if constexpr (W4Q) {
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
            b = dec4n<true>(w_at(cw[u], s));
          } else if constexpr (FMT == GF_SB) {
            b = dec4n<false>(w_at(cw[u], s));
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
            if constexpr (FMT == GF_W8)
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
            half4 a;
            if constexpr (FMT == GF_W4)
              a = xsel_w4x4(xv[u][t][0], xsel);
            else
              a = xperm_x4(make_uint2(xv[u][t][0].x, xv[u][t][0].y));
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
// chunks, lanes and groups of the streaming kernel
// ---------------------------------------------------------------------------
// A "chunk" is 16 bytes of codes per lane, 64 bytes per row (4 lanes), i.e.
// CK = 128 (int4), 64 (int8) or 32 (fp16) values of k.  A chunk holds GPC
// scale groups; before the MFMAs the four lanes of a row exchange words with
// v_permlane32_swap / v_permlane16_swap so that every MFMA's 32 (or 16) k
// belong to one group:
//   GPC = 2: swap32(w0,w2), swap32(w1,w3): lanes keep the half of each group
//            at k offsets {0,32,16,48}[kq] (int4) or {0,16,8,24}[kq] (int8);
//   GPC = 4: a 4x4 word transpose across the four lanes (two swap32, two
//            swap16): lane kq then holds word kq of every group.
// Codes decode into fp16 in natural k order, so activations are used as
// stored.  Codes and scales come through raw buffer loads (scalar base,
// 32-bit lane offset; an invalid chunk reads zeros through an out-of-range
// scalar offset, so the loop body has no branches).
template <int FMT, int G>
struct F2 {
  // NIB: symmetric codes whose low (or only) plane is int4 code words;
  // SYMS: one fp16 scale per (row, group); PLAIN: unscaled 16-bit weights;
  // HW: 32-bit words of the high plane per lane and chunk (6-bit 2, 5-bit 1)
  static constexpr bool NIB = FMT == GF_W4 || FMT == GF_W5 || FMT == GF_W6;
  static constexpr bool SYMS = NIB || FMT == GF_W8;
  static constexpr bool PLAIN = FMT == GF_F16 || FMT == GF_BF16;
  static constexpr int HW = FMT == GF_W6 ? 2 : (FMT == GF_W5 ? 1 : 0);
  static constexpr int CK = (NIB || FMT == GF_SB) ? 128 : (FMT == GF_W8 ? 64 : 32);
  static constexpr int GK = (FMT == GF_SB || PLAIN) ? 32 : G;
  static constexpr int GPC = CK / GK;
  static constexpr int KPM = (FMT == GF_W8 && G == 16) ? 16 : 32;  // k per MFMA
  static constexpr int MPG = GK / KPM;                             // MFMAs per group
  static constexpr int NM = GPC * MPG;                             // MFMAs per chunk
  static constexpr int XH = KPM / 4;                               // x halves per lane per MFMA
};

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// 4 int8 codes -> fp16 q in natural order (q + 128 lands in the mantissa of 1024)
__device__ __forceinline__ uint2 dec8n(uint32_t v) {
  const uint32_t u = v ^ 0x80808080u;
  const uint32_t lo = perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = perm(0x64646464u, u, 0x04030402u);
  return make_uint2(hsub2(lo, 0x64806480u), hsub2(hi, 0x64806480u));
}

// k offset (within the chunk) of the x values matching MFMA (g, p) on lane kq
template <int FMT, int G>
__device__ __forceinline__ int x_base(int kq) {
  typedef F2<FMT, G> F;
  if constexpr (F::GPC == 1) {
    if constexpr (F::PLAIN) return 8 * kq;
    return 16 * kq;  // int8 g64
  } else if constexpr (F::GPC == 2) {
    if constexpr (F::NIB) return (kq & 1) * 32 + (kq >> 1) * 16;
    return (kq & 1) * 16 + (kq >> 1) * 8;  // int8 g32
  } else {
    return kq * F::XH;  // int4 g32 / SB (8 k), int8 g16 (4 k)
  }
}
template <int FMT, int G>
constexpr int x_const(int g, int p) {
  typedef F2<FMT, G> F;
  if constexpr (F::GPC == 1) return F::PLAIN ? 0 : 8 * p;
  else if constexpr (F::GPC == 2) return F::NIB ? 64 * g + 8 * p : 32 * g;
  else return g * F::GK;
}


// bytes of LDS for a workgroup's activation slice: 80 KB keeps two
// workgroups per compute unit; an unsplit launch may take up to 150 KB (one
// per compute unit) rather than pay for a K split's partial tiles
constexpr int kXBudget = 80 * 1024;
constexpr int kXBudgetUnsplit = 150 * 1024;
// largest M that the two-range plan takes (two k ranges of up to 8 rows fill
// the 16 A rows)
constexpr int kRangesMaxM = 8;

// ---------------------------------------------------------------------------
// the streaming kernel: a workgroup = RT row tiles x one slice of K
// ---------------------------------------------------------------------------
// Every wave owns CPW chunks of one 16-row tile and issues its code and scale
// loads before it computes: all of them up to eight chunks (that keeps the most
// bytes in flight; vector loads of a wave complete in issue order, so nothing
// is loaded behind them), a window of eight for sixteen.  The workgroup's waves
// copy its slice of the activations (rows < M) into LDS with global_load_lds,
// a zero row stands for m >= M, and after one barrier the waves compute from
// LDS.  (An output row depends only on its own operand row, so rows >= M
// could read any row; reading row 0, or a zeroed region of one chunk, and not
// writing a whole zero row both measured 6-11% slower at M = 1.)
//
// K is cut into `split` slices of cps chunks.  The waves of a tile reduce
// through LDS in wave order; with split = 1 they store fp16, otherwise each
// workgroup stores its fp32 partial tile group in the workspace, and the
// `split` partials are added in slice order (deterministic, no floating-point
// atomics): by the last of the tile group's workgroups to finish, in the same
// launch, for up to kSplitInLaunch slices (split_arrive / split_finish), by a
// second kernel for more.  Splitting feeds the compute units when there
// are few row tiles, and keeps the LDS slice of x small when M * K is large;
// RT tiles per workgroup share one slice.
struct Split5 {
  int split;      // K slices
  int cps;        // chunks per slice
  int wpt;        // waves per row tile
  int rt;         // row tiles per workgroup
  int groups[3];  // tile groups (workgroups per slice) of each matrix
};

template <int FMT, int G>
struct CodeSlot {
  uint4 c;                              // codes (the low plane for W6 / W5)
  uint32_t s;                           // SB: d | dmin << 16
  uint32_t sub[FMT == GF_SB ? 3 : 1];   // SB: packed 6-bit sub-scale codes
  uint32_t hi[FMT == GF_W6 ? 2 : 1];    // W6 / W5: the high plane of the lane's four words
};

// High plane of one code word -> a word shaped like it: the high bits of the
// code in nibble i of each half sit in bits 0..1 of that nibble.  6-bit: hc
// is the word's uint16 (nibble i = hi(even) | hi(odd) << 2); 5-bit: its byte
// (bit i = hi(even), bit 4 + i = hi(odd)).
template <int FMT>
__device__ __forceinline__ uint32_t hi_spread(uint32_t hc) {
  if constexpr (FMT == GF_W6) {
    return (hc & 0x3333u) | ((hc & 0xccccu) << 14);
  } else {
    uint32_t x = (hc & 0x0fu) | ((hc & 0xf0u) << 12);  // bits 0-3 and 16-19
    x = (x | (x << 6)) & 0x03030303u;                  // -> bits 0,1,8,9 of each half
    return (x | (x << 3)) & 0x11111111u;               // -> bit 0 of each nibble
  }
}

// One int4 code word v plus its spread high bits h -> fp16 (u - 2^(b-1)) for
// k = 0..7 in natural order, u = nibble | hi << 4 (b = 6 or 5).  As in dec4n,
// nibbles 0 and 2 land in the mantissa of 1024 (ulp 1) and nibbles 1 and 3 in
// that of 64 (ulp 1/16); the high bits join them at bits 4..5 or 8..9, one
// AND-OR each, and one packed subtract removes 1024 + 2^(b-1) or 64 + 2^(b-1).
template <int BITS>
__device__ __forceinline__ half8 dec56(uint32_t v, uint32_t h) {
  constexpr uint32_t blo = BITS == 6 ? 0x64206420u : 0x64106410u;  // 1056 : 1040
  constexpr uint32_t bhi = BITS == 6 ? 0x56005600u : 0x55005500u;  // 96 : 80
  const uint32_t hl = h << 4, hr = h >> 4, v8 = v >> 8;
  const uint32_t o0 = and_or(hl, 0x00300030u, 0x64006400u);
  const uint32_t o1 = and_or(hl, 0x03000300u, 0x54005400u);
  const uint32_t o2 = and_or(hr, 0x00300030u, 0x64006400u);
  const uint32_t o3 = and_or(hr, 0x03000300u, 0x54005400u);
  const uint32_t h0 = hsub2(and_or(v, 0x000f000fu, o0), blo);
  const uint32_t h1 = hsub2(and_or(v, 0x00f000f0u, o1), bhi);
  const uint32_t h2 = hsub2(and_or(v8, 0x000f000fu, o2), blo);
  const uint32_t h3 = hsub2(and_or(v8, 0x00f000f0u, o3), bhi);
  return __builtin_bit_cast(half8, make_uint4(h0, h1, h2, h3));
}

// fp16 activations -> bf16 hi + lo with hi + lo exact: hi keeps the top 8
// significant bits (truncation of the fp32 value), lo = x - hi has at most 3
// and is exact in bf16.  Both products with bf16 weights are exact in fp32.
__device__ __forceinline__ void split_bf16(const half8& a, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float f = (float)a[i];
    const uint32_t fb = __float_as_uint(f) & 0xffff0000u;
    const float r = f - __uint_as_float(fb);
    hi[i] = __builtin_bit_cast(__bf16, (uint16_t)(fb >> 16));
    lo[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(r) >> 16));
  }
}

// MR: activation rows that can be non-zero among a lane's four outputs
// (m <= MR), so scale multiplications skip rows that are known to be zero.
//
// ST (streamed, 128-k chunks, one row tile, no split): instead of one
// activation slice shared through LDS, every wave copies the activations of
// its own chunks, one chunk at a time, into a private double buffer of 16 MT
// rows x 128 k (rows >= M in the last copied 4-row group read zeros through
// the buffer resource's range check; later groups are zeroed once and not
// copied), and computes chunk i while chunk i + 1 arrives.
// Rows are 256 bytes with the 16-byte segment s of row r stored at slot
// s ^ (r & 15), so the sixteen rows an MFMA operand read touches fall in
// distinct banks.  A workgroup then covers all of K for its 16 rows without a
// second, reducing launch, at any K; the cost is that each workgroup reads all
// of x.
//
// H = 2 (M <= 8, int4 groups; "k ranges"): a tile is R = 8 rows, and MFMA
// column c = h R + r holds row r over the h-th of two equal, contiguous
// halves of K, while A row a = h M + m holds activation row m over that same
// half (rows a >= 2 M read the zero row).  Output (h M + m, h R + r) is then
// row r's dot product with x_m over half h, the other outputs are discarded,
// and the two halves are added at the end.  The MFMA work per byte is
// unchanged (at M <= 8 at least half of the A rows are padding either way),
// but a matrix has twice as many tiles: one of 2048 rows fills 256
// workgroups, one per compute unit, without a K split.  In LDS each
// activation row takes cps * 128 + 16 halves and its second half sits 16
// bytes further along than a contiguous copy would put it, so the sixteen
// (m, h) pairs an operand read touches start 32 m + 16 h bytes into a bank
// row: all distinct.
// s_waitcnt vmcnt(n) for a wave-uniform n in 1..7 (0 above): the streamed
// activations' wait for one chunk's copies, whose count depends on M
__device__ __forceinline__ void wait_vm_st(int n) {
  switch (n) {
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
// ---------------------------------------------------------------------------
// K split added up inside the launch
// ---------------------------------------------------------------------------
// The `split` workgroups of a tile group (one per K slice) each store their
// fp32 partial tile with agent-scope stores, which are coherent across the
// XCDs' separate L2 caches, wait until those stores have completed, and then
// count themselves in on the tile group's counter.  The workgroup that arrives
// last reads the split partial tiles back with agent-scope loads, adds them in
// slice order (the same order, so the same bits, whichever workgroup arrives
// last) and stores fp16.  The increment wraps modulo split, so that last
// arrival also returns the counter to zero for the next call.  No cache-wide
// fence is needed (those write back or invalidate a whole XCD L2): the data
// itself is stored and loaded coherently, the counter is updated only after
// the stores completed, and the reads are issued only after the update returned.
// Up to kSplitInLaunch slices the last workgroup adds them; more slices
// leave more partial bytes to that one workgroup than a second, reducing
// kernel spread over the whole chip costs (measured: 4096x16384 at M = 16,
// eight slices, 16.4 us with the second kernel against 18.8 us in launch;
// four slices, 2048x8192 at M = 16 and 4096x16384 at M = 32: 8.6 -> 7.8 and
// 18.2 -> 17.0 us in launch).
constexpr int kSplitInLaunch = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSC1 = 16;  // cache-policy operand of the buffer builtins: sc1 (agent scope)
// buffer resource over the tile group's partial tiles, split * ent floats
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* part, int split, int ent) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)part, (short)0, split * ent * 4, 0x00020000);
}
// four consecutive outputs idx .. idx + 3 of slice s: stored coherently
// (agent scope) for the in-launch sums, plainly for the second kernel, which
// the kernel boundary orders after them
__device__ __forceinline__ void part_store4(__amdgpu_buffer_rsrc_t r, int s, int ent, int idx, float4v v,
                                            bool coherent) {
  // (whole-vector bit casts only: a bit cast of one vector element reads
  // element 0 with this compiler)
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  if (coherent)
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (uint32_t)idx * 4u, (uint32_t)(s * ent) * 4u, kSC1);
  else
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (uint32_t)idx * 4u, (uint32_t)(s * ent) * 4u, 0);
}
// true, in every thread, for the workgroup that arrives last at counter c;
// flag: an LDS word no thread reads or writes at this point
__device__ __forceinline__ bool split_arrive(uint32_t* c, int split, uint32_t* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __builtin_amdgcn_atomic_inc32(c, (uint32_t)(split - 1), __ATOMIC_RELAXED, "agent");
  __syncthreads();
  return *flag == (uint32_t)(split - 1);
}
// The last workgroup's sums: the tile group's ent outputs (RT tiles x MT
// activation tiles x 256), four consecutive ones per thread, every slice's
// load issued before the first add
template <int MT>
__device__ __forceinline__ void split_finish(__amdgpu_buffer_rsrc_t r, int split, int ent, int rt, int grp, int M,
                                             int ldy, const GemvMatrix& A) {
  constexpr int E = MT * 4 * 64;
  for (int i4 = threadIdx.x; i4 < ent / 4; i4 += blockDim.x) {
    float4v vals[16];
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
      if (s2 < split)
        vals[s2] = __builtin_bit_cast(
            float4v, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)i4 * 16u, (uint32_t)(s2 * ent) * 4u, kSC1));
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = vals[0][c];
#pragma unroll
    for (int s2 = 1; s2 < 16; ++s2)
      if (s2 < split)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] += vals[s2][c];
    const int idx = 4 * i4;
    const int rr = idx / E, e = idx - rr * E;
    const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
    const int m = t * 16 + 4 * (l >> 4) + q;
    const int nn = (grp * rt + rr) * 16 + (l & 15);
    if (m < M) {
      uint16_t* yr = A.y + (size_t)m * ldy;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (nn + c < A.n) yr[nn + c] = f32_to_f16_bits(v[c]);
    }
  }
}

// Streamed activations with two activation tiles run at most eight waves per
// workgroup (one row tile, at most 64 chunks in waves of 2, 4 or 8 chunks),
// so they declare 512 threads and get the register file of two waves per
// SIMD: declared for 1024, the compiler capped them at 128 VGPRs and spilled
// (4096x8192 at M = 32: int4 group 32 31.7 -> 13.7 us, 6-bit 33.1 -> 17.2,
// SB256 58.8 -> 41.9, int4 group 64 14.8 -> 13.4).
template <int FMT, int G, int MT, int CPW, int MR, bool ST = false, int H = 1>
__global__ void __launch_bounds__(ST && MT == 2 ? 512 : 1024) gemv5_kernel(const GemvBatch p, const Split5 sp) {
  typedef F2<FMT, G> F;
  typedef CodeSlot<FMT, G> S;
  static_assert(!ST || F::CK == 128, "streamed activations: 128-k chunks");
  static_assert(H == 1 || (MT == 1 && !ST && FMT == GF_W4 && H == 2), "k ranges: M <= 8, int4");
  constexpr int R = 16 / H;                                 // rows per tile
  constexpr int QN = MT == 1 ? (H * MR < 4 ? H * MR : 4) : 4;  // outputs per lane that are kept
  static_assert(FMT != GF_SB || CPW % 2 == 0, "SB256: a wave's chunks pair into superblocks");
  extern __shared__ uint4 lds4[];
  uint16_t* xl = (uint16_t*)lds4;

  // slice and tile group; every field of the three descriptors is read
  // unconditionally so picking the matrix costs no dependent scalar load
  const int gtot = sp.groups[0] + sp.groups[1] + sp.groups[2];
  const int s = blockIdx.x / gtot;
  const int gall = blockIdx.x - s * gtot;
  const int g0 = sp.groups[0], g1 = sp.groups[1];
  const bool in1 = gall >= g0, in2 = gall >= g0 + g1;
  const int grp = gall - (in2 ? g0 + g1 : (in1 ? g0 : 0));
  GemvMatrix A;
  A.codes = in2 ? p.mat[2].codes : (in1 ? p.mat[1].codes : p.mat[0].codes);
  A.scales = in2 ? p.mat[2].scales : (in1 ? p.mat[1].scales : p.mat[0].scales);
  A.mins = in2 ? p.mat[2].mins : (in1 ? p.mat[1].mins : p.mat[0].mins);
  A.sub = in2 ? p.mat[2].sub : (in1 ? p.mat[1].sub : p.mat[0].sub);
  A.x = in2 ? p.mat[2].x : (in1 ? p.mat[1].x : p.mat[0].x);
  A.y = in2 ? p.mat[2].y : (in1 ? p.mat[1].y : p.mat[0].y);
  A.n = in2 ? p.mat[2].n : (in1 ? p.mat[1].n : p.mat[0].n);
  A.tiles = in2 ? p.mat[2].tiles : (in1 ? p.mat[1].tiles : p.mat[0].tiles);

  const int NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = wave / sp.wpt;  // row tile of this wave within the group
  const int wv = wave - r * sp.wpt;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int kq = lane >> 4;
  const int tile = grp * sp.rt + r;
  const int k = p.k;
  const int M = p.m;
  const int nchunks = k / F::CK;
  const int kch = nchunks / H;         // chunks of one k range (H > 1: one slice)
  const int hr = H > 1 ? j / R : 0;    // this lane's k range
  const bool tvalid = H > 1 ? tile * R < A.n : tile < A.tiles;
  const int n = tile * R + (H > 1 ? j - hr * R : j);
  const bool nvalid = n < A.n;
  const int cbeg = s * sp.cps;
  const int cend = H > 1 ? kch : min(nchunks, cbeg + sp.cps);
  const int ldl = sp.cps * F::CK + (H > 1 ? 16 : 8);  // LDS row stride (halves)
  constexpr uint32_t kOOB = 0x7ffff000u;  // scalar offset past any buffer: loads read zero

  // buffer resources (num_records in bytes).  Rows >= n read row 0: their
  // output columns are never stored and MFMA columns are independent.
  const uint32_t rowbytes = (uint32_t)nchunks * 64u;
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc((void*)A.codes, (short)0, (int)((uint32_t)A.n * rowbytes), 0x00020000);
  const uint32_t coff = (nvalid ? (uint32_t)n * rowbytes : 0u) + (uint32_t)kq * 16u + (uint32_t)(hr * kch) * 64u;
  __amdgpu_buffer_rsrc_t rs = rc, rm = rc, rb = rc;
  uint32_t soff = 0, sboff = 0, subb = 0;
  // int8 group 64 stores 2 bytes of scales per chunk, so after a row with an
  // odd number of chunks the next row starts in the middle of a dword.  Such
  // a row loads its scale span from the dword below, one word longer, and
  // shifts it down 16 bits (sh16) before use: every dword the range check
  // sees is then aligned to the buffer, and only the buffer's last dword can
  // end past the (rounded-up) range.
  constexpr bool kHalfRow = F::SYMS && F::GPC == 1;
  uint32_t sh16 = 0;
  if constexpr (F::HW > 0) {
    const uint32_t hrow = (uint32_t)(k / 8) * (FMT == GF_W6 ? 2u : 1u);
    rb = __builtin_amdgcn_make_buffer_rsrc((void*)A.sub, (short)0, (int)((uint32_t)A.n * hrow), 0x00020000);
    subb = (nvalid ? (uint32_t)n * hrow : 0u) + (uint32_t)kq * (4u * F::HW);
  }
  if constexpr (F::SYMS) {
    // the range is rounded up to whole dwords: the range check zeroes a
    // dword that ends past it as a whole, and with an odd number of groups
    // per row (int8 group 64) and an odd number of rows the last scale shares
    // its dword with the two bytes after the buffer.  Those bytes lie in the
    // same aligned dword (the buffer starts 16-byte aligned), so never in
    // another page; like the next row's scales that a wave's span reaches,
    // they belong to chunks past the slice, whose scales are dropped.
    const uint32_t srow = (uint32_t)(k / F::GK) * 2u;
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)A.scales, (short)0, (int)(((uint32_t)A.n * srow + 3u) & ~3u),
                                           0x00020000);
    soff = (nvalid ? (uint32_t)n * srow : 0u) + (uint32_t)(hr * kch) * (F::GPC * 2u);
    if constexpr (kHalfRow) {
      sh16 = (soff & 2u) << 3;
      soff &= ~3u;
    }
  } else if constexpr (FMT == GF_SB) {
    const uint32_t nsb = (uint32_t)(k / 256);
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)A.scales, (short)0, (int)((uint32_t)A.n * nsb * 2u), 0x00020000);
    rm = __builtin_amdgcn_make_buffer_rsrc((void*)A.mins, (short)0, (int)((uint32_t)A.n * nsb * 2u), 0x00020000);
    rb = __builtin_amdgcn_make_buffer_rsrc((void*)A.sub, (short)0, (int)((uint32_t)A.n * nsb * 12u), 0x00020000);
    sboff = nvalid ? (uint32_t)n * nsb * 2u : 0u;
    subb = nvalid ? (uint32_t)n * nsb * 12u : 0u;
  }

  // 1. the workgroup's activation slice: rows < M, 64 blocks of 8 halves per
  //    copy instruction, copy instructions dealt round-robin to the waves.
  //    The copies are LDS DMA reads written as inline asm: the compiler,
  //    which cannot tell which LDS bytes a DMA writes, would otherwise wait
  //    for every load in flight (the code loads included) before the first
  //    LDS read.  They write no register.  The issue loop is the copy's cost
  //    at M = 32 (a workgroup issues M * K / 512 of them), so it walks
  //    (row, block) with increments and no per-copy division or lane test
  //    when every copy is whole.  For two activation tiles (M > 16) the code
  //    loads, which come from HBM and take longer, go out first so that their
  //    latency covers that loop; for one tile the copies go out first and
  //    each chunk's compute waits only for its own code load.
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;
  auto copy_x = [&]() {
    const int blocks = (H > 1 ? nchunks : cend - cbeg) * (F::CK / 8);
    const int per_row = (blocks + 63) >> 6;
    if constexpr (H > 1) {
      // k ranges (one slice, whole 1 KB blocks): copies (m, col) dealt
      // round-robin to the waves; the second half's blocks (col >= kch / 4)
      // land 16 bytes further
      const int bpr = kch / 4;
      const uint32_t lrow = (uint32_t)ldl * 2u, grow = (uint32_t)p.ldx * 2u;
      const uint8_t* xs = (const uint8_t*)A.x + lane * 16;
      int m = 0, col = wave;
      while (col >= per_row) {
        col -= per_row;
        ++m;
      }
      while (m < M) {
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(xs + (uint32_t)m * grow + (uint32_t)col * 1024u),
                        "s"(lds_base + (uint32_t)m * lrow + (uint32_t)col * 1024u + (col >= bpr ? 16u : 0u))
                     : "memory", "m0");
        col += NW;
        while (col >= per_row) {
          col -= per_row;
          ++m;
        }
      }
      for (int b = threadIdx.x; b < blocks; b += blockDim.x) *(uint4*)(xl + M * ldl + b * 8) = make_uint4(0u, 0u, 0u, 0u);
      return;
    }
    if constexpr (MR == 1) {  // one activation row (M = 1): wave w copies blocks w, w + NW, ...
      const uint8_t* xs = (const uint8_t*)(A.x + (size_t)cbeg * F::CK) + lane * 16;
      for (int col = wave; col < per_row; col += NW)
        if (col * 64 + lane < blocks)
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :: "v"(xs + col * 1024), "s"(lds_base + (uint32_t)col * 1024u) : "memory", "m0");
      for (int b = threadIdx.x; b < blocks; b += blockDim.x) *(uint4*)(xl + ldl + b * 8) = make_uint4(0u, 0u, 0u, 0u);
      return;
    }
    int m, col, dm, dc;
    if ((per_row & (per_row - 1)) == 0) {  // the usual case: shifts, no division
      const int sh = __builtin_ctz((unsigned)per_row);
      m = wave >> sh;
      col = wave & (per_row - 1);
      dm = NW >> sh;
      dc = NW & (per_row - 1);
    } else {
      m = wave / per_row;
      col = wave - m * per_row;
      dm = NW / per_row;
      dc = NW - dm * per_row;
    }
    const uint32_t lrow = (uint32_t)ldl * 2u;     // LDS bytes per row
    const uint32_t grow = (uint32_t)p.ldx * 2u;   // global bytes per row (M * ldx < 2^31)
    const uint8_t* xs = (const uint8_t*)(A.x + (size_t)cbeg * F::CK) + lane * 16;
    uint32_t goff = (uint32_t)m * grow + (uint32_t)col * 1024u;  // byte offsets of this copy
    uint32_t loff = lds_base + (uint32_t)m * lrow + (uint32_t)col * 1024u;
    const uint32_t gstep = (uint32_t)dm * grow + (uint32_t)dc * 1024u;
    const uint32_t lstep = (uint32_t)dm * lrow + (uint32_t)dc * 1024u;
    const uint32_t gwrap = grow - (uint32_t)per_row * 1024u, lwrap = lrow - (uint32_t)per_row * 1024u;
#define RQ_COPY_STEP                                   \
  col += dc;                                           \
  m += dm;                                             \
  goff += gstep;                                       \
  loff += lstep;                                       \
  if (col >= per_row) {                                \
    col -= per_row;                                    \
    ++m;                                               \
    goff += gwrap;                                     \
    loff += lwrap;                                     \
  }
    if ((blocks & 63) == 0) {
      while (m < M) {
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(xs + goff), "s"(loff) : "memory", "m0");
        RQ_COPY_STEP
      }
    } else {
      while (m < M) {
        if (col * 64 + lane < blocks)
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :: "v"(xs + goff), "s"(loff) : "memory", "m0");
        RQ_COPY_STEP
      }
    }
#undef RQ_COPY_STEP
    for (int b = threadIdx.x; b < blocks; b += blockDim.x) *(uint4*)(xl + M * ldl + b * 8) = make_uint4(0u, 0u, 0u, 0u);
  };
  constexpr bool kCodesFirst = MT == 2;
  if constexpr (!kCodesFirst && !ST) copy_x();

  // 2. this wave's scales and codes: all of them, or for sixteen chunks at
  //    M <= 2 a window of eight, the next issued as each chunk is computed.
  //    (With all sixteen issued at once a wave reaches its first chunk's math
  //    only once its last load has issued, when most of its bytes have
  //    arrived; the window made 4096x16384 at M = 1 and 2 8% faster.)
  //    Chunks outside the slice (or of a tile past the matrix) read zero
  //    codes; their scales are zeroed after loading (the scale span is read
  //    in one piece and may run into the next slice or row)
  const int c0 = cbeg + wv * CPW;
  S sl[CPW];
  constexpr int SW = F::SYMS ? (CPW * F::GPC * 2 + 3) / 4 + (kHalfRow ? 1 : 0) : 1;  // scale words
  uint32_t sw[SW];
  if constexpr (F::SYMS) {
    const uint32_t ss = tvalid ? (uint32_t)c0 * (F::GPC * 2) : kOOB;
#pragma unroll
    for (int q = 0; q < SW / 4; ++q) {
      auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, soff, ss + 16u * q, 0);
      sw[4 * q] = t[0]; sw[4 * q + 1] = t[1]; sw[4 * q + 2] = t[2]; sw[4 * q + 3] = t[3];
    }
    constexpr int B = SW / 4 * 4;
    if constexpr (SW % 4 == 3) {
      auto t = __builtin_amdgcn_raw_buffer_load_b96(rs, soff, ss + 4u * B, 0);
      sw[B] = t[0]; sw[B + 1] = t[1]; sw[B + 2] = t[2];
    } else if constexpr (SW % 4 == 2) {
      auto t = __builtin_amdgcn_raw_buffer_load_b64(rs, soff, ss + 4u * B, 0);
      sw[B] = t[0]; sw[B + 1] = t[1];
    } else if constexpr (SW % 4 == 1) {
      sw[B] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, ss + 4u * B, 0);
    }
  }
  auto load_chunk = [&](int i) {
    const int c = c0 + i;
    const bool valid = tvalid && c < cend;
    auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, coff, valid ? (uint32_t)c * 64u : kOOB, 0);
    sl[i].c = make_uint4(v[0], v[1], v[2], v[3]);
    if constexpr (F::HW == 2) {
      auto h = __builtin_amdgcn_raw_buffer_load_b64(rb, subb, valid ? (uint32_t)c * 32u : kOOB, 0);
      sl[i].hi[0] = h[0];
      sl[i].hi[1] = h[1];
    } else if constexpr (F::HW == 1) {
      sl[i].hi[0] = __builtin_amdgcn_raw_buffer_load_b32(rb, subb, valid ? (uint32_t)c * 16u : kOOB, 0);
    }
    if constexpr (FMT == GF_SB) {
      // a superblock is two chunks and a wave's chunk range starts even (CPW
      // and the slice length are even): load its scales once, with the pair's
      // first chunk
      if (i & 1) return;
      const uint32_t sb = (uint32_t)c >> 1;
      const uint32_t s2 = valid ? sb * 2u : kOOB;
      const uint32_t s12 = valid ? sb * 12u : kOOB;
      const uint32_t d = __builtin_amdgcn_raw_buffer_load_b16(rs, sboff, s2, 0);
      const uint32_t dm = __builtin_amdgcn_raw_buffer_load_b16(rm, sboff, s2, 0);
      sl[i].s = d | (dm << 16);
      auto t = __builtin_amdgcn_raw_buffer_load_b96(rb, subb, s12, 0);
      sl[i].sub[0] = t[0];
      sl[i].sub[1] = t[1];
      sl[i].sub[2] = t[2];
    }
  };
  constexpr int RD = (CPW == 16 && MR <= 2 && !ST && !kCodesFirst) ? 8 : CPW;  // loads in flight
#pragma unroll
  for (int i = 0; i < RD; ++i) load_chunk(i);

  // keep everything that uses the loaded scales below this point: hoisted
  // between the loads, it would wait for the scale load before the first
  // code load is issued
  __builtin_amdgcn_sched_barrier(0);

  // 3. wait for this wave's copies.  Copies first: with at most RD loads
  //    still in flight, every DMA issued before the RD code loads has landed
  //    (a wave's vector loads complete in issue order), and each chunk below
  //    waits only for its own code load.  Codes first: everything.  Then a
  //    plain barrier.
  // streamed: this wave's buffers and the copy of one chunk (4 MT DMA reads
  // of 4 rows x 256 bytes; lane l: row 4q + l / 16, slot l % 16)
  constexpr int kStBuf = 16 * MT * 128 * 2;  // bytes per buffer
  constexpr int kStCopies = 4 * MT;          // DMA reads per chunk
  const uint32_t st_lds = lds_base + (uint32_t)wave * (2u * kStBuf);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)A.x, (short)0, (int)((uint32_t)M * (uint32_t)p.ldx * 2u), 0x00020000);
  const uint32_t st_r = (uint32_t)(lane >> 4), st_s = (uint32_t)(lane & 15);
  // only the 4-row groups that hold rows < M are copied (a group past M would
  // read zeros through the range check); the others are zeroed once in both
  // buffers.  4096x16384 at M = 4 and 8: 15.6 and 15.8 -> 14.4 and 15.4 us
  const int st_nq = (M + 3) >> 2 < kStCopies ? (M + 3) >> 2 : kStCopies;
  auto st_copy = [&](int i) {  // chunk c0 + i (clamped inside the slice) into buffer i & 1
    const int c = c0 + i < cend ? c0 + i : cend - 1;
#pragma unroll
    for (int q = 0; q < kStCopies; ++q) {
      if (q >= st_nq) break;
      const uint32_t r = 4u * q + st_r;
      const uint32_t voff = r * (uint32_t)p.ldx * 2u + (uint32_t)c * 256u + ((st_s ^ (r & 15u)) << 4);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :: "v"(voff), "s"(rx), "s"(st_lds + (uint32_t)(i & 1) * kStBuf + 1024u * q) : "memory", "m0");
    }
  };
  if constexpr (ST) {
    for (int q = st_nq; q < kStCopies; ++q) {
      *(uint4*)((uint8_t*)lds4 + wave * 2 * kStBuf + 1024 * q + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)((uint8_t*)lds4 + wave * 2 * kStBuf + kStBuf + 1024 * q + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
    }
    st_copy(0);
    if (CPW > 1) st_copy(1);
  } else if constexpr (kCodesFirst) {
    copy_x();
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    // with a high plane two loads follow per chunk: every copy has landed
    // once no more than 2 * RD are in flight
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(F::HW > 0 ? 2 * RD : RD) : "memory");
  }

  int xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = t * 16 + j;
    if constexpr (H > 1) {  // A row j = h M + m < 2 M: row m, half h; the others the zero row
      const int h = j / M;
      xrow[t] = (j < H * M ? (j - h * M) * ldl + h * (kch * F::CK + 8) : M * ldl) + x_base<FMT, G>(kq);
    } else {
      xrow[t] = (m < M ? m : M) * ldl + x_base<FMT, G>(kq);
    }
  }
  float4v acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kHalfRow) {
#pragma unroll
    for (int i = 0; i + 1 < SW; ++i) sw[i] = __builtin_amdgcn_alignbit(sw[i + 1], sw[i], sh16);
  }

  // 4. compute, chunk by chunk
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const bool valid = tvalid && c0 + i < cend;
    const int c = c0 + i < cend ? c0 + i : cend - 1;  // activation offset inside the slice
    const int kk = (c - cbeg) * F::CK;
    if constexpr (RD < CPW) {
      if (i + RD < CPW) load_chunk(i + RD);
      __builtin_amdgcn_sched_barrier(0);  // keep the load here, ahead of this chunk's math
    }
    if constexpr (ST) {
      // chunk i has landed once only chunk i + 1's copies may be in flight
      if (i + 1 < CPW) wait_vm_st(st_nq);
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    uint32_t w[4] = {sl[i].c.x, sl[i].c.y, sl[i].c.z, sl[i].c.w};
    uint32_t gw[4][2], gh[4][2];
    // the high plane's words go through the same exchange as the code words
    uint32_t hw[4] = {0u, 0u, 0u, 0u};
    if constexpr (F::HW == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) hw[j] = hi_spread<FMT>((sl[i].hi[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    } else if constexpr (F::HW == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) hw[j] = hi_spread<FMT>((sl[i].hi[0] >> (8 * j)) & 0xffu);
    }
    if constexpr (F::GPC == 2) {
      swap32(w[0], w[2]);
      swap32(w[1], w[3]);
      gw[0][0] = w[0]; gw[0][1] = w[1];
      gw[1][0] = w[2]; gw[1][1] = w[3];
      if constexpr (F::HW > 0) {
        swap32(hw[0], hw[2]);
        swap32(hw[1], hw[3]);
        gh[0][0] = hw[0]; gh[0][1] = hw[1];
        gh[1][0] = hw[2]; gh[1][1] = hw[3];
      }
    } else if constexpr (F::GPC == 4) {
      swap32(w[0], w[2]);
      swap32(w[1], w[3]);
      swap16(w[0], w[1]);
      swap16(w[2], w[3]);
      gw[0][0] = w[0]; gw[1][0] = w[1]; gw[2][0] = w[2]; gw[3][0] = w[3];
      if constexpr (F::HW > 0) {
        swap32(hw[0], hw[2]);
        swap32(hw[1], hw[3]);
        swap16(hw[0], hw[1]);
        swap16(hw[2], hw[3]);
        gh[0][0] = hw[0]; gh[1][0] = hw[1]; gh[2][0] = hw[2]; gh[3][0] = hw[3];
      }
    }
    float scl[4], mnv[4];
    if constexpr (F::SYMS) {
#pragma unroll
      for (int g = 0; g < F::GPC; ++g) {
        const int h = i * F::GPC + g;  // half-word index in the wave's scale span
        const uint32_t word = sw[h >> 1];
        const float v = f16_bits_to_f32((uint16_t)((h & 1) ? (word >> 16) : (word & 0xffffu)));
        scl[g] = valid ? v : 0.f;
      }
    } else if constexpr (FMT == GF_SB) {
      const S& sp2 = sl[i & ~1];  // the superblock's scales, loaded with its first chunk
      const float d = f16_bits_to_f32((uint16_t)(sp2.s & 0xffffu));
      const float dm = f16_bits_to_f32((uint16_t)(sp2.s >> 16));
      const uint64_t lo48 = (uint64_t)sp2.sub[0] | ((uint64_t)(sp2.sub[1] & 0xffffu) << 32);
      const uint64_t hi48 = (uint64_t)(sp2.sub[1] >> 16) | ((uint64_t)sp2.sub[2] << 16);
      const int half = (c & 1) * 4;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        scl[g] = d * (float)((uint32_t)(lo48 >> (6 * (half + g))) & 63u);  // exact
        mnv[g] = dm * (float)((uint32_t)(hi48 >> (6 * (half + g))) & 63u);
      }
    }
#pragma unroll
    for (int g = 0; g < F::GPC; ++g) {
      float4v grp[MT], xs[MT];
#pragma unroll
      for (int pp = 0; pp < F::MPG; ++pp) {
        const int xo = kk + x_const<FMT, G>(g, pp);
        if constexpr (F::KPM == 32) {
          half8 b;
          if constexpr (F::PLAIN) {
            b = __builtin_bit_cast(half8, make_uint4(w[0], w[1], w[2], w[3]));  // bf16 bits for GF_BF16
          } else if constexpr (FMT == GF_W4 || FMT == GF_SB) {
            b = dec4n<FMT == GF_W4>(F::GPC == 2 ? gw[g][pp] : gw[g][0]);
          } else if constexpr (F::HW > 0) {
            b = dec56<FMT == GF_W6 ? 6 : 5>(F::GPC == 2 ? gw[g][pp] : gw[g][0], F::GPC == 2 ? gh[g][pp] : gh[g][0]);
          } else {
            uint32_t wa, wb;
            if constexpr (F::GPC == 1) {
              wa = w[2 * pp];
              wb = w[2 * pp + 1];
            } else {
              wa = gw[g][0];
              wb = gw[g][1];
            }
            const uint2 lo = dec8n(wa), hi = dec8n(wb);
            b = __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            half8 a;
            if constexpr (ST) {
              // row t * 16 + j of buffer i & 1, segment (x offset / 8) at slot seg ^ j
              const int seg = (x_base<FMT, G>(kq) + x_const<FMT, G>(g, pp)) >> 3;
              a = *(const half8*)(xl + ((i & 1) * kStBuf + wave * 2 * kStBuf) / 2 + (t * 16 + j) * 128 +
                                  ((seg ^ j) << 3));
            } else {
              a = *(const half8*)(xl + xrow[t] + xo);
            }
            if constexpr (FMT == GF_F16) {
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
            } else if constexpr (FMT == GF_BF16) {
              bf16x8 ahi, alo;
              split_bf16(a, ahi, alo);
              const bf16x8 wb = __builtin_bit_cast(bf16x8, b);
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, wb, acc[t], 0, 0, 0);
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, wb, acc[t], 0, 0, 0);
            } else {
              grp[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, pp == 0 ? zero4 : grp[t], 0, 0, 0);
              if constexpr (FMT == GF_SB) {
                const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
                xs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, zero4, 0, 0, 0);
              }
            }
          }
        } else {
          const uint2 rr = dec8n(gw[g][0]);
          const half4 b = __builtin_bit_cast(half4, rr);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const half4 a = *(const half4*)(xl + xrow[t] + xo);
            grp[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, zero4, 0, 0, 0);
          }
        }
      }
      if constexpr (!F::PLAIN) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int q = 0; q < QN; ++q) {
            acc[t][q] += scl[g] * grp[t][q];
            if constexpr (FMT == GF_SB) acc[t][q] -= mnv[g] * xs[t][q];
          }
      }
    }
    if constexpr (ST) {
      // buffer i & 1 is free once this chunk's reads have returned
      if (i + 2 < CPW) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        st_copy(i + 2);
      }
    }
  }

  // 5. reduce the waves of each row tile in wave order
  float (*red)[MT][4][64] = (float (*)[MT][4][64])lds4;
  __syncthreads();  // everyone is done with the activations
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][t][q][lane] = acc[t][q];
  __syncthreads();
  if constexpr (H > 1) {
    // (m, row r of tile rr): output (h M + m, h R + r) summed over the
    // halves h, each over the tile's waves in wave order
    const int per_tile = M * R;
    for (int idx = threadIdx.x; idx < sp.rt * per_tile; idx += blockDim.x) {
      const int rr = idx / per_tile, e = idx - rr * per_tile;
      const int m = e / R, rw = e - m * R;
      float v = 0.f;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int a = h * M + m;
        const int l = (a >> 2) * 16 + h * R + rw;
        for (int w2 = 0; w2 < sp.wpt; ++w2) v += red[rr * sp.wpt + w2][0][a & 3][l];
      }
      const int nn = (grp * sp.rt + rr) * R + rw;
      if (nn < A.n) A.y[(size_t)m * p.ldy + nn] = f32_to_f16_bits(v);
    }
    return;
  }
  constexpr int E = MT * 4 * 64;  // outputs of one row tile (rows m < 16 MT)
  const int ent = sp.rt * E;
  if (sp.split > 1) {
    // four consecutive outputs per thread (same row tile, activation tile
    // and q; lanes l .. l + 3)
    const __amdgpu_buffer_rsrc_t rp = part_rsrc(p.ws + (size_t)gall * sp.split * ent, sp.split, ent);
    for (int i4 = threadIdx.x; i4 < ent / 4; i4 += blockDim.x) {
      const int idx = 4 * i4;
      const int rr = idx / E, e = idx - rr * E;
      const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
      float4v v = *(const float4v*)&red[rr * sp.wpt][t][q][l];
      for (int w2 = 1; w2 < sp.wpt; ++w2) {
        const float4v u = *(const float4v*)&red[rr * sp.wpt + w2][t][q][l];
        v[0] += u[0];
        v[1] += u[1];
        v[2] += u[2];
        v[3] += u[3];
      }
      part_store4(rp, s, ent, idx, v, sp.split <= kSplitInLaunch);
    }
    if (sp.split <= kSplitInLaunch && split_arrive(p.cnt + gall, sp.split, (uint32_t*)lds4))
      split_finish<MT>(rp, sp.split, ent, sp.rt, grp, M, p.ldy, A);
    return;
  }
  for (int idx = threadIdx.x; idx < ent; idx += blockDim.x) {
    const int rr = idx / E, e = idx - rr * E;
    const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
    float v = red[rr * sp.wpt][t][q][l];
    for (int w2 = 1; w2 < sp.wpt; ++w2) v += red[rr * sp.wpt + w2][t][q][l];
    const int m = t * 16 + 4 * (l >> 4) + q;
    const int nn = (grp * sp.rt + rr) * 16 + (l & 15);
    if (m < M && nn < A.n) A.y[(size_t)m * p.ldy + nn] = f32_to_f16_bits(v);
  }
}

// Split K over more than kSplitInLaunch slices, second step: y = fp16(sum of
// the `split` partial tiles, in slice order), one thread per output of a tile
// group.  The kernel boundary orders it after every slice's stores.
template <int MT>
__global__ void __launch_bounds__(256) gemv5_reduce_kernel(const GemvBatch p, const Split5 sp) {
  constexpr int E = MT * 4 * 64;
  const int ent = sp.rt * E;
  const int gtot = sp.groups[0] + sp.groups[1] + sp.groups[2];
  // block b = j * gtot + gall sums outputs j * 256 ... of tile group gall
  // (ent is a multiple of 256).  Workgroups are dealt to the eight XCDs
  // round-robin, so with gtot % 8 == 0 this block runs on the XCD whose L2
  // holds the partial tiles (written by blocks s * gtot + gall).
  const int j = __builtin_amdgcn_readfirstlane((int)blockIdx.x / gtot);
  const int gall = (int)blockIdx.x - j * gtot;
  if (j * 256 >= ent) return;
  const int idx = j * 256 + (int)threadIdx.x;
  // every slice's load is issued before the first add (slices past the split
  // read zero through an out-of-range offset); the adds run in slice order
  constexpr uint32_t kOOB = 0x7ffff000u;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ws + (size_t)gall * sp.split * ent), (short)0, (int)(sp.split * ent * 4), 0x00020000);
  float vals[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2)
    vals[s2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rw, (uint32_t)idx * 4u, s2 < sp.split ? (uint32_t)(s2 * ent) * 4u : kOOB, 0));
  float v = vals[0];
#pragma unroll
  for (int s2 = 1; s2 < 16; ++s2)
    if (s2 < sp.split) v += vals[s2];
  const int g0 = sp.groups[0], g1 = sp.groups[1];
  const bool in1 = gall >= g0, in2 = gall >= g0 + g1;
  const int grp = gall - (in2 ? g0 + g1 : (in1 ? g0 : 0));
  const GemvMatrix& A = p.mat[in2 ? 2 : (in1 ? 1 : 0)];
  const int rr = idx / E, e = idx - rr * E;
  const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
  const int m = t * 16 + 4 * (l >> 4) + q;
  const int nn = (grp * sp.rt + rr) * 16 + (l & 15);
  if (m < p.m && nn < A.n) A.y[(size_t)m * p.ldy + nn] = f32_to_f16_bits(v);
}

// ---------------------------------------------------------------------------
// phased activations: a workgroup = RT row tiles x a slice of K, the slice's
// activations, codes and scales streamed through LDS in phases
// ---------------------------------------------------------------------------
// For batches that fill two activation tiles, staging a workgroup's whole
// activation slice before any math (the streaming kernel above) either caps
// the slice at what LDS holds, so that K is split into many slices whose
// fp32 partial tiles must all be added, or (one row tile per workgroup)
// makes every workgroup read all of x.  Here the slice is cut into phases of
// P = 4 chunks (512 k), each moved into one of NB LDS buffers (three for two
// activation tiles, four for one) by LDS DMA reads, NB - 1 phases ahead: the
// 16 MT activation rows (1 KB each; rows >= M read zeros through the buffer
// resource's range check), the RT x 16 code rows (256 bytes each) and their
// scales.  The reads of a phase are dealt evenly over every wave of the
// workgroup (one wave issuing them all was limited by its issue rate), and
// the math reads only LDS.  At phase q every wave waits for its own reads of
// phase q (those of later phases may stay in flight); one barrier then makes
// the buffer visible and tells that every wave is done with phase q - 1,
// whose buffer receives phase q + NB - 1.  All RT row tiles read the same
// activation rows, so x crosses L2 once per RT tiles, and the whole K of
// most matrices fits one slice.
//
// Each of eight waves owns one eighth of every phase's (chunk, group) pairs
// for two row tiles: it reads an activation fragment from LDS once and
// multiplies it into both, so LDS delivers a phase's activations once per
// two tiles rather than once per tile.  With four row tiles the workgroup
// runs sixteen waves, the second eight on tiles 2 and 3: four waves per
// SIMD hide the LDS and MFMA latencies of the short per-phase chains better
// than two (width-4096 shapes at M = 12..32: 2-6% faster; at two tiles,
// sixteen waves of one tile each were 1% slower).  A lane reads from LDS
// exactly the code words the streaming kernel's lane exchange would hand it
// (the 8 k at the fragment's offset), so no exchange is needed.  The eight
// partial sums of each output (one per pair share) are added through LDS in
// share order at the end.  Activation rows are padded to 1040 bytes and the 16-byte segments of
// code row r are stored at slot (segment ^ (r % 16)), so the sixteen rows of
// an operand read fall in distinct banks.  Decode and scaling are those of
// the streaming kernel (symmetric int4).
struct Plan6 {
  int split;      // K slices (partial tiles added in launch up to kSplitInLaunch, else by gemv5_reduce_kernel)
  int cps;        // chunks per slice, a multiple of 4
  int groups[3];  // tile groups (of RT tiles) per matrix
};

template <int G, int MT, int RT>
struct G6 {
  static constexpr int P = 4;                    // chunks per phase
  static constexpr int NB = MT == 1 ? 4 : 3;     // LDS buffers (phases in flight + 1)
  static constexpr int NWP = 8;                  // waves sharing out a phase's (chunk, group) pairs
  static constexpr int TS = RT >= 4 ? 2 : 1;     // row-tile shares (sixteen waves for four tiles)
  static constexpr int NW = NWP * TS;            // waves
  static constexpr int RTW = RT / TS;            // row tiles of a wave
  static constexpr int GPC = 128 / G;            // scale groups per chunk
  static constexpr int PPW = P * GPC / NWP;      // (chunk, group) pairs of a wave per phase
  static constexpr int RS = P * 256 + 16;        // LDS bytes per activation row
  static constexpr int XR = 16 * MT;             // activation rows (one DMA each)
  static constexpr int CD = RT * P;              // code DMAs (4 rows x 256 bytes each)
  static constexpr int SR = RT * 16 > 64 ? RT * 16 : 64;  // scale rows held (one DMA per 64)
  static constexpr int SP = 64 / G;              // 16-byte parts of a row's phase span
  static constexpr int SD = SP * (SR / 64);      // scale DMAs per phase
  static constexpr int ND = XR + CD + SD;        // DMA reads per phase
  static constexpr int DPW = (ND + NW - 1) / NW; // per wave, at most
  static constexpr int XB = XR * RS;
  static constexpr int CB = RT * 16 * P * 64;
  static constexpr int SB = SP * SR * 16;        // scale spans: [SP][SR rows][16 bytes]
  static constexpr int BUF = XB + CB + SB;
  static constexpr size_t LDS = (size_t)NB * BUF;
  static_assert(PPW >= 1 && P * GPC == PPW * NWP, "the pairs of a phase");
  static_assert(RTW >= 1 && RT == TS * RTW, "the row-tile shares");
  static_assert(SR % 64 == 0 && SR >= RT * 16, "the scale DMAs cover the code rows");
  static_assert(NB * BUF >= (size_t)NWP * RT * MT * 1024, "the reduction fits the buffers");
  static_assert((NB - 1) * DPW <= 63, "the phases in flight within the wait counter");
};

// s_waitcnt vmcnt(n) for a uniform n in 0..63 (the counter's range)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
    case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
    case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
    case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
    case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
    case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
    case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
    case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
    case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
    case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
    case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
    case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
    case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
    case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
    case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
    case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
    case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
    case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
    case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
    case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
    case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
    case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
    case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
    case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
    case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
  }
}

template <int G, int MT, int RT>
__global__ void __launch_bounds__(RT >= 4 ? 1024 : 512) gemv6_kernel(const GemvBatch p, const Plan6 sp) {
  typedef F2<GF_W4, G> F;
  typedef G6<G, MT, RT> C;
  constexpr int P = C::P, NB = C::NB, RS = C::RS, BUF = C::BUF, DPW = C::DPW;
  extern __shared__ uint4 lds4[];

  const int gtot = sp.groups[0] + sp.groups[1] + sp.groups[2];
  const int s = blockIdx.x / gtot;
  const int gall = blockIdx.x - s * gtot;
  const int g0 = sp.groups[0], g1 = sp.groups[1];
  const bool in1 = gall >= g0, in2 = gall >= g0 + g1;
  const int grp = gall - (in2 ? g0 + g1 : (in1 ? g0 : 0));
  GemvMatrix A;
  A.codes = in2 ? p.mat[2].codes : (in1 ? p.mat[1].codes : p.mat[0].codes);
  A.scales = in2 ? p.mat[2].scales : (in1 ? p.mat[1].scales : p.mat[0].scales);
  A.x = in2 ? p.mat[2].x : (in1 ? p.mat[1].x : p.mat[0].x);
  A.y = in2 ? p.mat[2].y : (in1 ? p.mat[1].y : p.mat[0].y);
  A.n = in2 ? p.mat[2].n : (in1 ? p.mat[1].n : p.mat[0].n);
  A.tiles = in2 ? p.mat[2].tiles : (in1 ? p.mat[1].tiles : p.mat[0].tiles);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int k = p.k;
  const int M = p.m;
  const int nchunks = k / 128;
  const int cbeg = s * sp.cps;
  const int cend = min(nchunks, cbeg + sp.cps);
  const int nph = (cend - cbeg) / P;
  constexpr uint32_t kOOB = 0x7ffff000u;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;
  const uint32_t rowbytes = (uint32_t)nchunks * 64u;
  const uint32_t srow = (uint32_t)(k / G) * 2u;

  // this wave's DMA reads of a phase: d = wave DPW + i over the list
  // [activation rows 0 .. XR - 1][code DMAs 0 .. CD - 1][scale spans]; a code
  // DMA e covers group rows 4e .. 4e + 3 (lane l -> row 4e + l / 16, LDS slot
  // l % 16 holding segment (l % 16) ^ (row % 16)); scale span u: lane l ->
  // row l, 16 bytes at u 16 of its phase span.  The lane's byte offset at the
  // slice's first phase (kOOB past the data: the read returns zeros) stays in
  // a register; a phase adds its offset through the scalar offset operand.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A.x, (short)0, (int)(((uint32_t)(M - 1) * (uint32_t)p.ldx + (uint32_t)k) * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc((void*)A.codes, (short)0, (int)((uint32_t)A.n * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A.scales, (short)0, (int)(((uint32_t)A.n * srow + 3u) & ~3u), 0x00020000);
  const int d0 = wave * DPW;
  const int nmine = max(0, min(DPW, C::ND - d0));
  uint32_t vo[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int d = d0 + i;
    if (d < C::XR) {
      vo[i] = d < M ? (uint32_t)d * (uint32_t)p.ldx * 2u + (uint32_t)cbeg * 256u + (uint32_t)lane * 16u : kOOB;
    } else if (d < C::XR + C::CD) {
      const int row = 4 * (d - C::XR) + (lane >> 4);
      const int nn = grp * RT * 16 + row;
      const int seg = (lane & 15) ^ (row & 15);
      vo[i] = nn < A.n ? (uint32_t)nn * rowbytes + (uint32_t)cbeg * 64u + (uint32_t)seg * 16u : kOOB;
    } else {
      // scale DMA u: span part u % SP of rows 64 (u / SP) + lane
      const int u = d - C::XR - C::CD;
      const int part = u % C::SP, row = (u / C::SP) * 64 + lane;
      const int nn = grp * RT * 16 + row;
      vo[i] = (row < RT * 16 && nn < A.n)
                  ? (uint32_t)nn * srow + (uint32_t)cbeg * (F::GPC * 2u) + (uint32_t)part * 16u
                  : kOOB;
    }
  }
  auto dma = [&](int q, int b) {
    const uint32_t bb = lds_base + (uint32_t)(b * BUF);
    const uint32_t qx = (uint32_t)q * (P * 256u), qc = (uint32_t)q * (P * 64u), qs = (uint32_t)q * (P * F::GPC * 2u);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int d = d0 + i;
      if (d < C::XR) {
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :: "v"(vo[i]), "s"(rx), "s"(qx), "s"(bb + (uint32_t)(d * RS)) : "memory", "m0");
      } else if (d < C::XR + C::CD) {
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :: "v"(vo[i]), "s"(rc), "s"(qc), "s"(bb + (uint32_t)(C::XB + (d - C::XR) * 1024))
                     : "memory", "m0");
      } else if (d < C::ND) {
        const int u = d - C::XR - C::CD;
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :: "v"(vo[i]), "s"(rsc), "s"(qs),
                        "s"(bb + (uint32_t)(C::XB + C::CB + ((u % C::SP) * C::SR + (u / C::SP) * 64) * 16))
                     : "memory", "m0");
      }
    }
  };

  const int j = lane & 15;
  const int kq = lane >> 4;
  // wave = th NWP + pw: pair share pw of every phase, row tiles th RTW ..
  const int th = wave / C::NWP, pw = wave - th * C::NWP;
  bool tv[C::RTW];
#pragma unroll
  for (int r = 0; r < C::RTW; ++r) tv[r] = grp * RT + th * C::RTW + r < A.tiles;

  float4v acc[C::RTW][MT];
#pragma unroll
  for (int r = 0; r < C::RTW; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = float4v{0.f, 0.f, 0.f, 0.f};
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* lds8 = (const uint8_t*)lds4;

  auto compute = [&](int b) {
    const uint8_t* bufp = lds8 + b * BUF;
    const uint8_t* xb = bufp + j * RS + x_base<GF_W4, G>(kq) * 2;
#pragma unroll
    for (int e = 0; e < C::PPW; ++e) {
      const int pi = pw * C::PPW + e;
      const int ci = pi / C::GPC, g = pi - ci * C::GPC;  // chunk within the phase, group
      // the lane's code bytes for k step pp: at ci 64 + (k offset of its
      // fragment) / 2 within the row's phase span
      const int b0 = ci * 64 + (x_base<GF_W4, G>(kq) + x_const<GF_W4, G>(g, 0)) / 2;
      half8 af[F::MPG][MT];
#pragma unroll
      for (int pp = 0; pp < F::MPG; ++pp) {
        const int xo = (ci * 128 + x_const<GF_W4, G>(g, pp)) * 2;
#pragma unroll
        for (int t = 0; t < MT; ++t) af[pp][t] = *(const half8*)(xb + t * 16 * RS + xo);
      }
      const int hh = ci * C::GPC + g;  // scale half-word of the phase span
#pragma unroll
      for (int r = 0; r < C::RTW; ++r) {
        const int row = (th * C::RTW + r) * 16 + j;
        const uint8_t* cr = bufp + C::XB + row * 256 + (b0 & 15);
        uint32_t wv[2];
        if constexpr (F::MPG == 2) {
          const uint2 u = *(const uint2*)(cr + (((b0 >> 4) ^ j) << 4));
          wv[0] = u.x;
          wv[1] = u.y;
        } else {
          wv[0] = *(const uint32_t*)(cr + (((b0 >> 4) ^ j) << 4));
          wv[1] = 0u;
        }
        const uint32_t word = *(const uint32_t*)(bufp + C::XB + C::CB + (hh >> 3) * (C::SR * 16) + row * 16 +
                                                 ((hh & 7) >> 1) * 4);
        const float v = f16_bits_to_f32((uint16_t)((hh & 1) ? (word >> 16) : (word & 0xffffu)));
        const float scl = tv[r] ? v : 0.f;
        float4v grp4[MT];
#pragma unroll
        for (int pp = 0; pp < F::MPG; ++pp) {
          const half8 bq = dec4n<true>(wv[pp]);
#pragma unroll
          for (int t = 0; t < MT; ++t)
            grp4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[pp][t], bq, pp == 0 ? zero4 : grp4[t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][t][q] += scl * grp4[t][q];
      }
    }
  };

#pragma unroll
  for (int q = 0; q < NB - 1; ++q)
    if (q < nph) dma(q, q);
  for (int q = 0; q < nph; ++q) {
    // this wave's reads of phase q have landed once only those of the later
    // phases already issued (up to NB - 2) are in flight
    wait_vm(nmine * min(NB - 2, nph - 1 - q));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (q + NB - 1 < nph) dma(q + NB - 1, (q + NB - 1) % NB);
    compute(q % NB);
  }

  // the NWP pair shares' partial sums of each output, added in share order
  constexpr int E = MT * 4 * 64;  // outputs of one row tile (rows m < 16 MT)
  const int ent = RT * E;
  float (*red)[RT][MT][4][64] = (float (*)[RT][MT][4][64])lds4;
  __syncthreads();  // every wave is done with the buffers
#pragma unroll
  for (int r = 0; r < C::RTW; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[pw][th * C::RTW + r][t][q][lane] = acc[r][t][q];
  __syncthreads();
  if (sp.split > 1) {
    // four consecutive outputs per thread (lanes l .. l + 3)
    const __amdgpu_buffer_rsrc_t rp = part_rsrc(p.ws + (size_t)gall * sp.split * ent, sp.split, ent);
    for (int i4 = threadIdx.x; i4 < ent / 4; i4 += blockDim.x) {
      const int idx = 4 * i4;
      const int rr = idx / E, e = idx - rr * E;
      const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
      float4v v = *(const float4v*)&red[0][rr][t][q][l];
#pragma unroll
      for (int w2 = 1; w2 < C::NWP; ++w2) {
        const float4v u = *(const float4v*)&red[w2][rr][t][q][l];
        v[0] += u[0];
        v[1] += u[1];
        v[2] += u[2];
        v[3] += u[3];
      }
      part_store4(rp, s, ent, idx, v, sp.split <= kSplitInLaunch);
    }
    if (sp.split <= kSplitInLaunch && split_arrive(p.cnt + gall, sp.split, (uint32_t*)lds4))
      split_finish<MT>(rp, sp.split, ent, RT, grp, M, p.ldy, A);
    return;
  }
  for (int idx = threadIdx.x; idx < ent; idx += blockDim.x) {
    const int rr = idx / E, e = idx - rr * E;
    const int t = e >> 8, q = (e >> 6) & 3, l = e & 63;
    float v = red[0][rr][t][q][l];
#pragma unroll
    for (int w2 = 1; w2 < C::NWP; ++w2) v += red[w2][rr][t][q][l];
    const int m = t * 16 + 4 * (l >> 4) + q;
    const int nn = (grp * RT + rr) * 16 + (l & 15);
    if (m < M && nn < A.n) A.y[(size_t)m * p.ldy + nn] = f32_to_f16_bits(v);
  }
}

// Launch shape of gemv6_kernel, or false to leave the product to the
// streaming kernel: four row tiles per workgroup (x then crosses L2 twice
// per code byte at M = 32, within what a compute unit reads from L2 while its
// codes stream from HBM) and K slices of whole phases until there is a
// workgroup per compute unit.
struct Shape6 {
  int rt;
  Plan6 plan;
};
constexpr int kG6Rt = 4;

static bool plan6(const GemvBatch& b, int group, int min_m, Shape6& sh) {
  const int nchunks = b.k / 128;
  if (b.m < min_m || nchunks == 0 || nchunks % 4 != 0) return false;
  // an activation slice that fits one workgroup's LDS whole: the streaming
  // kernel stages it once, unsplit, unless four row tiles on sixteen waves
  // take it (checked below)
  const bool fits_unsplit = (size_t)(b.m + 1) * (size_t)(b.k + 8) * 2u <= (size_t)kXBudgetUnsplit;
  constexpr size_t kLim = (size_t)1 << 31;
  for (int i = 0; i < b.nmat; ++i) {
    const size_t n = (size_t)b.mat[i].n;
    if (n * (size_t)nchunks * 64u >= kLim || n * (size_t)(b.k / group) * 2u >= kLim) return false;
  }
  if ((size_t)b.m * (size_t)b.ldx * 2u >= kLim) return false;
  int tiles = 0;
  for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
  // one activation tile's streamed plan of the streaming kernel (192 to 256
  // row tiles, at most 64 chunks) does better without a K split
  if (tiles >= 192 && tiles <= 256 && nchunks <= 64) return false;
  auto groups = [&](int r) {
    int g = 0;
    for (int i = 0; i < b.nmat; ++i) g += (b.mat[i].tiles + r - 1) / r;
    return g;
  };
  const int nph = nchunks / 4;
  // slices of whole phases until there are 192 workgroups
  auto slices = [&](int r, int& cps_out) {
    int sp = 1;
    while (groups(r) * sp < 192 && sp < 16 && nph >= 4 * sp) sp *= 2;
    cps_out = (nph + sp - 1) / sp * 4;
    return (nchunks + cps_out - 1) / cps_out;
  };
  int rt = kG6Rt, cps = 0;
  int split = slices(rt, cps);
  // two row tiles per workgroup where four would need more slices than the
  // launch adds up itself and two do not (2048x8192 at M = 32: four tiles
  // in 8 slices plus the reducing kernel 9.37 us, two in 4 slices 9.12; at
  // M = 17 9.35 against 8.92), at the price of twice the activation reads
  if (split > kSplitInLaunch) {
    int cps2 = 0;
    const int split2 = slices(2, cps2);
    if (split2 <= kSplitInLaunch && groups(2) * split2 >= 192) {
      rt = 2;
      split = split2;
      cps = cps2;
    }
  }
  const int mt = b.m <= 16 ? 1 : 2;
  if (groups(rt) * split < 192) return false;
  // four row tiles on sixteen waves, unsplit, beat the streaming kernel's
  // unsplit slice (K = 4096 at M = 9..17: 16384x4096 13.5-16.8 -> 11.9-13.7
  // us, 12288x4096 12.6-15.5 -> 11.1-12.9); with K split to fill the chip
  // (6144x2048, 8192x2048, 10240x2560) or on two tiles they do not
  // (6144x2048 at M = 32: 7.4 -> 8.8 us)
  if (fits_unsplit && (rt != kG6Rt || split != 1)) return false;
  if (split > 1 && (!b.ws || (split <= kSplitInLaunch && (!b.cnt || groups(rt) > kSplitCounters)) ||
                    (size_t)groups(rt) * split * rt * mt * 1024 > b.ws_bytes))
    return false;
  sh.rt = rt;
  sh.plan.split = split;
  sh.plan.cps = cps;
  for (int i = 0; i < 3; ++i) sh.plan.groups[i] = i < b.nmat ? (b.mat[i].tiles + rt - 1) / rt : 0;
  return true;
}

template <int G>
static bool launch6(const GemvBatch& b, const Shape6& sh, hipStream_t st, hipError_t& err) {
  const int mt = b.m <= 16 ? 1 : 2;
  const int gtot = sh.plan.groups[0] + sh.plan.groups[1] + sh.plan.groups[2];
  err = hipSuccess;
  if (gtot == 0) return true;
  const dim3 grid((unsigned)(gtot * sh.plan.split));
#define RQ_L6(MT, RT)                                                                                \
  do {                                                                                               \
    typedef G6<G, MT, RT> C6;                                                                        \
    static_assert(C6::LDS <= (size_t)160 * 1024, "LDS of a compute unit");                           \
    static const bool attr_set = hipFuncSetAttribute((const void*)gemv6_kernel<G, MT, RT>,             \
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,      \
                                                     (int)C6::LDS) == hipSuccess;                    \
    (void)attr_set;                                                                                  \
    hipLaunchKernelGGL((gemv6_kernel<G, MT, RT>), grid, dim3(C6::NW * 64), C6::LDS, st, b, sh.plan);   \
  } while (0)
  if (sh.rt == 2) {
    if (mt == 2) RQ_L6(2, 2); else RQ_L6(1, 2);
  } else {
    if (mt == 2) RQ_L6(2, kG6Rt); else RQ_L6(1, kG6Rt);
  }
#undef RQ_L6
  err = hipGetLastError();
  if (err == hipSuccess && sh.plan.split > kSplitInLaunch) {
    Split5 sp5;
    sp5.split = sh.plan.split;
    sp5.cps = sh.plan.cps;
    sp5.wpt = 1;
    sp5.rt = sh.rt;
    for (int i = 0; i < 3; ++i) sp5.groups[i] = sh.plan.groups[i];
    const int outs = gtot * sh.rt * mt * 256;
    const dim3 rgrid((unsigned)((outs + 255) / 256));
    if (mt == 2)
      hipLaunchKernelGGL(gemv5_reduce_kernel<2>, rgrid, dim3(256), 0, st, b, sp5);
    else
      hipLaunchKernelGGL(gemv5_reduce_kernel<1>, rgrid, dim3(256), 0, st, b, sp5);
    err = hipGetLastError();
  }
  return true;
}

// Chunks per wave for a slice of `cps` chunks: a wave keeps CPW code loads in
// flight and a workgroup is best at four to eight waves per row tile, so the
// count grows with the slice (16 only for one activation tile and formats
// whose per-chunk operands fit the registers without spilling; from 64
// chunks at M = 1, where sixteen keep a window of eight loads: 2048x8192
// 6.49 -> 6.21 us).
static int pick_cpw(int cps, bool allow16, int m) {
  if (allow16 && (cps >= 128 || (m == 1 && cps >= 64))) return 16;
  return cps >= 32 ? 8 : 4;
}

// Launch shape for gemv5_kernel, or false when none fits (activation slice
// too large for LDS even at the finest split, or no workspace for a split).
// Preference: the fewest slices that give at least one workgroup per compute
// unit; then as many row tiles per workgroup (up to 4, sharing the x slice)
// as still keep that many workgroups.
template <int FMT, int G>
static bool plan5(const GemvBatch& b, Split5& sp, int& cpw_out, bool& stream_out, int& ranges_out) {
  typedef F2<FMT, G> F;
  const int nchunks = b.k / F::CK;
  const int mt = b.m <= 16 ? 1 : 2;
  bool found = false;
  stream_out = false;
  ranges_out = 1;
  // the kernel addresses every buffer through a buffer resource with a 32-bit
  // size and 32-bit offsets: each must stay below 2 GiB
  constexpr size_t kLim = (size_t)1 << 31;
  for (int i = 0; i < b.nmat; ++i) {
    const size_t n = (size_t)b.mat[i].n;
    if (n * (size_t)nchunks * 64u >= kLim) return false;
    if (F::SYMS && n * (size_t)(b.k / F::GK) * 2u >= kLim) return false;
    if (FMT == GF_SB && n * (size_t)(b.k / 256) * 12u >= kLim) return false;
    if (F::HW > 0 && n * (size_t)(b.k / 8) * 2u >= kLim) return false;
  }
  if ((size_t)b.m * (size_t)b.ldx * 2u >= kLim) return false;
  // M <= 8, int4 groups, fewer than 256 row tiles and at least 32 chunks:
  // two k ranges per 8-row tile, twice the workgroups without a split (the
  // kernel's H = 2).  Measured at M = 1: cmix value 2048x8192 6.37 -> 5.63
  // us; O 2048x2048 (16 chunks) 3.66 -> 3.85 us, and matrices of 256 row
  // tiles or more 4-10% slower, so those keep one range.  SB256 codes on two
  // ranges (whole superblocks per range) were slower than their four-slice
  // plan: 2560x10240 at M = 1 and 4, 11.4 and 12.6 -> 12.2 and 18.5 us
  if constexpr (FMT == GF_W4) {
    int tiles = 0;
    for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
    const size_t xb = (size_t)(b.m + 1) * (nchunks * F::CK + 16) * 2;
    const int kch = nchunks / 2;
    const int cpw = b.m <= 2 ? pick_cpw(kch, true, b.m) : (kch <= 24 ? 4 : 8);
    const int wpt = (kch + cpw - 1) / cpw;
    if (b.m <= kRangesMaxM && tiles < 256 && nchunks >= 32 && nchunks % 8 == 0 && xb <= (size_t)kXBudgetUnsplit &&
        wpt <= 16) {
      sp.split = 1;
      sp.cps = nchunks;
      sp.wpt = wpt;
      sp.rt = 1;
      for (int i = 0; i < 3; ++i) sp.groups[i] = i < b.nmat ? (b.mat[i].n + 7) / 8 : 0;
      cpw_out = cpw;
      ranges_out = 2;
      return true;
    }
  }
  // formats whose decode costs more per byte than int4 groups (SB256, 5-/6-bit
  // codes, int8 group 16), on fewer than 256 row tiles with a long K at
  // M <= 4: four K slices of waves of four chunks, for four times the
  // workgroups (2560x10240 at M = 1 and 4: 5-12% faster than one slice)
  constexpr bool kHeavy = FMT == GF_SB || F::HW > 0 || (FMT == GF_W8 && G == 16);
  if constexpr (kHeavy) {
    int tiles = 0;
    for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
    constexpr int cmult = ((F::GPC == 1 && F::SYMS) || FMT == GF_SB) ? 2 : 1;
    const int cps = ((nchunks + 3) / 4 + cmult - 1) / cmult * cmult;
    const int used = (nchunks + cps - 1) / cps;
    const int wpt = (cps + 3) / 4;
    const size_t xb = (size_t)(b.m + 1) * (cps * F::CK + 8) * 2;
    if (b.ws && b.cnt && b.m <= 4 && tiles < 256 && nchunks >= 64 && wpt <= 16 && xb <= (size_t)kXBudget &&
        (size_t)tiles * used * mt * 1024 <= b.ws_bytes) {
      sp.split = used;
      sp.cps = cps;
      sp.wpt = wpt;
      sp.rt = 1;
      for (int i = 0; i < 3; ++i) sp.groups[i] = i < b.nmat ? b.mat[i].tiles : 0;
      cpw_out = 4;
      return true;
    }
  }
  // an activation slice that does not fit one workgroup's LDS: stream it per
  // wave (one row tile per workgroup, waves of 2, 4 or 8 chunks) rather than
  // split K, when that makes 192 to 256 workgroups (one per CU) and the
  // waves' buffers fit.  Preferred for two activation tiles (M > 16) and
  // codes other than SB256 (against the split plan, 4096 rows at M = 32:
  // int4 group 64 K = 4096 7.65 vs 9.04 us, K = 8192 13.44 vs 13.77; int4
  // group 32 K = 4096 8.11 vs 9.74; SB256 K = 8192 41.9 vs 16.8).  With one
  // activation tile (M = 4..8) the split plan, whose slices are added in the
  // launch, is faster (4096x16384, int4 group 64 at M = 4, 6, 8: 13.58,
  // 13.29, 14.51 against 13.85, 14.82, 14.91 us streamed; group 32 at M = 4
  // 14.94 against 17.22; SB256 19.2 against 53.0), so there the streamed
  // plan serves only where no split is possible (no workspace, or none
  // found).  With fewer row tiles (2048x8192, 128) the split plan is faster,
  // since each workgroup streams all of x through one CU.
  bool stream_ok = false;
  Split5 streamed;
  int streamed_cpw = 0;
  if constexpr (F::CK == 128) {
    int tiles = 0;
    for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
    const size_t xb = (size_t)(b.m + 1) * (nchunks * F::CK + 8) * 2;
    if (xb > (size_t)kXBudgetUnsplit && (mt == 2 || b.m <= 8) && nchunks <= 64 * (3 - mt) && tiles >= 192 &&
        tiles <= 256) {
      const int cpw = nchunks <= 16 ? 2 : (nchunks <= 32 ? 4 : 8);
      streamed.split = 1;
      streamed.cps = nchunks;
      streamed.wpt = (nchunks + cpw - 1) / cpw;
      streamed.rt = 1;
      for (int i = 0; i < 3; ++i) streamed.groups[i] = i < b.nmat ? b.mat[i].tiles : 0;
      streamed_cpw = cpw;
      stream_ok = true;
      if (!b.ws || (mt == 2 && FMT != GF_SB)) {
        sp = streamed;
        cpw_out = cpw;
        stream_out = true;
        return true;
      }
    }
  }
  // row tiles share a workgroup (and its activation slice) only where that
  // slice is larger than the tile's codes, 16 rows x 64 bytes per chunk
  const bool share_x = (b.m + 1) * F::CK * 2 > 16 * 64;
  Split5 unsplit;
  int unsplit_cpw = 0;
  bool have_unsplit = false;
  // unsplit with a large activation slice, if that occupies at least half
  // of the compute units
  {
    const size_t xb = (size_t)(b.m + 1) * (nchunks * F::CK + 8) * 2;
    // two activation tiles over a short K: eight waves of two chunks issue
    // the activation copies twice as fast as four of four
    const int cpw = (mt == 2 && nchunks <= 16) ? 2 : pick_cpw(nchunks, mt == 1 && FMT != GF_SB && F::HW == 0, b.m);
    const int wpt = (nchunks + cpw - 1) / cpw;
    int tiles = 0;
    for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
    if (xb > (size_t)kXBudget && xb <= (size_t)kXBudgetUnsplit && wpt <= 16 && tiles >= 128) {
      int rt = 1;
      auto groups = [&](int r) {
        int g = 0;
        for (int i = 0; i < b.nmat; ++i) g += (b.mat[i].tiles + r - 1) / r;
        return g;
      };
      // down to 256 workgroups; to 128 while each still fetches more than
      // five times its codes' bytes of activations
      auto x_heavy = [&](int r) { return xb > (size_t)5 * r * 16 * 64 * nchunks; };
      while (share_x && rt < 4 && 2 * rt * wpt <= 16 &&
             (groups(2 * rt) >= 256 || (groups(2 * rt) >= 128 && x_heavy(rt))))
        rt *= 2;
      // such a slice leaves room for one workgroup per compute unit, so more
      // than 256 workgroups run in two rounds, the second partial: share more
      // tiles while at least 128 workgroups remain (fused R/K/V 3 x 4096^2
      // at M = 9, 12, 16: 13.2, 13.7, 14.1 -> 11.9, 12.1, 12.4 us)
      while (rt < 4 && 2 * rt * wpt <= 16 && groups(rt) > 256 && groups(2 * rt) >= 128) rt *= 2;
      // still more than 256 makes two rounds of one workgroup per CU: a K
      // split with small slices does better (10240x2560 at M = 16, 5-/6-bit
      // codes and SB256: 15.1-16.8 -> 14.4-15.6 us), where the stream has
      // the workspace for it
      Split5 u;
      u.split = 1;
      u.cps = nchunks;
      u.wpt = wpt;
      u.rt = rt;
      for (int i = 0; i < 3; ++i) u.groups[i] = i < b.nmat ? (b.mat[i].tiles + rt - 1) / rt : 0;
      if (groups(rt) <= 256 || !b.ws) {
        sp = u;
        cpw_out = cpw;
        return true;
      }
      // kept in case the workspace is too small for any split
      unsplit = u;
      unsplit_cpw = cpw;
      have_unsplit = true;
    }
  }
  for (int split = 1; split <= 16; split *= 2) {
    if (split > nchunks) break;
    if (split > 1 && !b.ws) break;
    // a wave's scale span is loaded from byte c0 * 2 * GPC and must start on a
    // 4-byte boundary: with one scale per chunk (int8 group 64) slices hold an
    // even number of chunks (CPW is even).  SB256 slices are even too, so a
    // wave's chunk pairs are whole superblocks.
    constexpr int cmult = ((F::GPC == 1 && F::SYMS) || FMT == GF_SB) ? 2 : 1;
    const int cps = ((nchunks + split - 1) / split + cmult - 1) / cmult * cmult;
    // slices of cps chunks that are not empty (fewer than split where the
    // rounding of cps leaves the last ones with nothing: 41 chunks in 8
    // slices of 6 make 7)
    const int used = (nchunks + cps - 1) / cps;
    const size_t xb = (size_t)(b.m + 1) * (cps * F::CK + 8) * 2;
    if (xb > (size_t)kXBudget) continue;
    // from M = 3 on: waves of four chunks for slices of up to 24, of eight
    // above (4096-wide matrices, 32 chunks, at M = 3..8: 3-19% faster than
    // four)
    // int8 group 16 (sixteen 16-k MFMAs per chunk) keeps waves of four chunks
    // up to 48 (width 2560 at M = 1 and 4: 6-7% faster than eight)
    constexpr int kCpw4Max = (FMT == GF_W8 && G == 16) ? 48 : 24;
    const int cpw = (FMT == GF_W8 && G == 16 && cps <= kCpw4Max) ? 4
                    : b.m <= 2 ? pick_cpw(cps, FMT != GF_SB && F::HW == 0, b.m) : (cps <= kCpw4Max ? 4 : 8);
    const int wpt = (cps + cpw - 1) / cpw;
    if (wpt > 16) continue;
    int rt = 1;
    auto groups = [&](int r) {
      int g = 0;
      for (int i = 0; i < b.nmat; ++i) g += (b.mat[i].tiles + r - 1) / r;
      return g;
    };
    // row tiles share a workgroup while the workgroups would not all be
    // resident at once (each CU holds as many as its 160 KB of LDS and its
    // waves allow), or while the activation slice outweighs four times the
    // group's codes and at least 256 workgroups remain.  Measured: fused
    // R/K/V 3x4096^2 at M = 4 8.7 us with one tile per workgroup (768, three
    // per CU) against 10.3 with two; cmix value 2048x8192 at M = 32 (K in
    // 8 slices) 10.0 us with four tiles against 10.7 with two.
    auto one_round = [&](int r) {
      const size_t red = (size_t)r * wpt * mt * 1024;
      const size_t lds = xb > red ? xb : red;
      const int by_lds = (int)((size_t)(160 * 1024) / lds);
      const int by_waves = (mt == 1 ? 32 : 24) / (r * wpt);
      return (size_t)groups(r) * used <= (size_t)256 * (by_lds < by_waves ? by_lds : by_waves);
    };
    auto x_heavy = [&](int r) { return xb > (size_t)4 * r * 16 * 64 * cps; };
    while (share_x && rt < 4 && 2 * rt * wpt <= 16 &&
           (!one_round(rt) || (x_heavy(rt) && groups(2 * rt) * used >= 256)))
      rt *= 2;
    if (used > 1 && (size_t)groups(rt) * rt * used * mt * 1024 > b.ws_bytes) break;
    // slices added in the launch need a counter per tile group; past that,
    // a larger split adds them in a second kernel
    if (used > 1 && used <= kSplitInLaunch && (!b.cnt || groups(rt) > kSplitCounters)) continue;
    sp.split = used;
    sp.cps = cps;
    sp.wpt = wpt;
    sp.rt = rt;
    for (int i = 0; i < 3; ++i) sp.groups[i] = i < b.nmat ? (b.mat[i].tiles + rt - 1) / rt : 0;
    cpw_out = cpw;
    found = true;
    // a split costs the partial tiles' round trip through the workspace and
    // the last workgroups' sums: worth it only to occupy more than half of
    // the compute units, or to fit the activations
    if (groups(rt) * used >= (used == 1 ? 128 : 256)) break;
  }
  if (!found && have_unsplit) {
    sp = unsplit;
    cpw_out = unsplit_cpw;
    return true;
  }
  if (!found && stream_ok) {
    sp = streamed;
    cpw_out = streamed_cpw;
    stream_out = true;
    return true;
  }
  return found;
}

// Dynamic LDS of a gemv5_kernel launch: the activation slice (or the waves'
// streamed buffers), or the reduction of the waves' partial tiles.
template <int FMT, int G>
static size_t lds5(const GemvBatch& b, const Split5& sp, bool stream, int ranges) {
  typedef F2<FMT, G> F;
  const int mt = b.m <= 16 ? 1 : 2;
  const int nw = sp.rt * sp.wpt;
  const size_t xb = stream ? (size_t)nw * 2 * (16 * mt * 128 * 2)
                           : (size_t)(b.m + 1) * (sp.cps * F::CK + (ranges > 1 ? 16 : 8)) * 2;
  const size_t red = (size_t)nw * mt * 4 * 64 * 4;
  return xb > red ? xb : red;
}

template <int FMT, int G>
static bool launch5(const GemvBatch& b, hipStream_t st, hipError_t& err) {
  typedef F2<FMT, G> F;
  Split5 sp;
  int cpw = 4;
  bool stream = false;
  int ranges = 1;
  if (!plan5<FMT, G>(b, sp, cpw, stream, ranges)) return false;
  const int mt = b.m <= 16 ? 1 : 2;
  const int nw = sp.rt * sp.wpt;
  const size_t lds = lds5<FMT, G>(b, sp, stream, ranges);
  const int gtot = sp.groups[0] + sp.groups[1] + sp.groups[2];
  err = hipSuccess;
  if (gtot == 0) return true;
  const dim3 grid((unsigned)(gtot * sp.split)), block((unsigned)(nw * 64));
#define RQ_L5(MT, CPW, MR)                                                                        \
  do {                                                                                            \
    static const bool attr_set =                                                                  \
        hipFuncSetAttribute((const void*)gemv5_kernel<FMT, G, MT, CPW, MR>,                       \
                            hipFuncAttributeMaxDynamicSharedMemorySize, kXBudgetUnsplit + 1024) == \
        hipSuccess;                                                                               \
    (void)attr_set;                                                                               \
    hipLaunchKernelGGL((gemv5_kernel<FMT, G, MT, CPW, MR>), grid, block, lds, st, b, sp);         \
  } while (0)
#define RQ_L5S(MT, CPW)                                                                           \
  do {                                                                                            \
    static const bool attr_set =                                                                  \
        hipFuncSetAttribute((const void*)gemv5_kernel<FMT, G, MT, CPW, 4, true>,                  \
                            hipFuncAttributeMaxDynamicSharedMemorySize, kXBudgetUnsplit + 1024) == \
        hipSuccess;                                                                               \
    (void)attr_set;                                                                               \
    hipLaunchKernelGGL((gemv5_kernel<FMT, G, MT, CPW, 4, true>), grid, block, lds, st, b, sp);    \
  } while (0)
  if constexpr (F::CK == 128) {
    if (stream) {
      // the kernel's declared bound for two activation tiles
      if (mt == 2 && nw > 8) {
        err = hipErrorInvalidConfiguration;
        return true;
      }
      if (mt == 2) {
        if (cpw == 2) RQ_L5S(2, 2); else if (cpw == 4) RQ_L5S(2, 4); else RQ_L5S(2, 8);
      } else {
        if (cpw == 2) RQ_L5S(1, 2); else if (cpw == 4) RQ_L5S(1, 4); else RQ_L5S(1, 8);
      }
      err = hipGetLastError();
      return true;
    }
  }
#undef RQ_L5S
#define RQ_L5H(CPW, MR)                                                                           \
  do {                                                                                            \
    static const bool attr_set =                                                                  \
        hipFuncSetAttribute((const void*)gemv5_kernel<FMT, G, 1, CPW, MR, false, 2>,              \
                            hipFuncAttributeMaxDynamicSharedMemorySize, kXBudgetUnsplit + 1024) == \
        hipSuccess;                                                                               \
    (void)attr_set;                                                                               \
    hipLaunchKernelGGL((gemv5_kernel<FMT, G, 1, CPW, MR, false, 2>), grid, block, lds, st, b, sp); \
  } while (0)
  if constexpr (FMT == GF_W4) {
    if (ranges == 2) {
      if (b.m == 1) {
        if (cpw == 4) RQ_L5H(4, 1); else if (cpw == 8) RQ_L5H(8, 1); else RQ_L5H(16, 1);
      } else if (b.m == 2) {
        if (cpw == 4) RQ_L5H(4, 2); else if (cpw == 8) RQ_L5H(8, 2); else RQ_L5H(16, 2);
      } else {
        if (cpw == 4) RQ_L5H(4, 4); else RQ_L5H(8, 4);
      }
      err = hipGetLastError();
      return true;
    }
  }
#undef RQ_L5H
  if (mt == 2) {
    if (cpw == 2) RQ_L5(2, 2, 4); else if (cpw == 4) RQ_L5(2, 4, 4); else RQ_L5(2, 8, 4);
  } else if constexpr (FMT == GF_SB || F::HW > 0) {
    if (b.m == 1) {
      if (cpw == 4) RQ_L5(1, 4, 1); else RQ_L5(1, 8, 1);
    } else if (b.m == 2) {
      if (cpw == 4) RQ_L5(1, 4, 2); else RQ_L5(1, 8, 2);
    } else {
      if (cpw == 4) RQ_L5(1, 4, 4); else RQ_L5(1, 8, 4);
    }
  } else if (b.m == 1) {
    if (cpw == 4) RQ_L5(1, 4, 1); else if (cpw == 8) RQ_L5(1, 8, 1); else RQ_L5(1, 16, 1);
  } else if (b.m == 2) {
    if (cpw == 4) RQ_L5(1, 4, 2); else if (cpw == 8) RQ_L5(1, 8, 2); else RQ_L5(1, 16, 2);
  } else {
    if (cpw == 4) RQ_L5(1, 4, 4); else if (cpw == 8) RQ_L5(1, 8, 4); else RQ_L5(1, 16, 4);
  }
#undef RQ_L5
  err = hipGetLastError();
  if (err == hipSuccess && sp.split > kSplitInLaunch) {
    const int outs = gtot * sp.rt * mt * 256;
    const dim3 rgrid((unsigned)((outs + 255) / 256));
    if (mt == 2)
      hipLaunchKernelGGL(gemv5_reduce_kernel<2>, rgrid, dim3(256), 0, st, b, sp);
    else
      hipLaunchKernelGGL(gemv5_reduce_kernel<1>, rgrid, dim3(256), 0, st, b, sp);
    err = hipGetLastError();
  }
  return true;
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// The phased kernel's shape for int4 groups, or false: past 16 activation
// rows wherever plan6 finds one; from 9 to 16 rows only where the streaming
// kernel would cut K into more slices than its launch adds up (a second,
// reducing kernel), or finds no plan, and the phased kernel needs no more
// slices than that
// (4096x16384 at M = 9, 12, 16: 15.8, 16.3, 16.3 -> 14.3, 14.6, 14.6 us;
// where the streaming kernel's split stays in its launch it is faster:
// 2048x8192 at M = 12, 16 7.4, 7.6 against 7.9, 8.0 us).
template <int FMT, int G>
static bool choose6(const GemvBatch& b, Shape6& sh) {
  if (b.k % 512 != 0) return false;
  if (plan6(b, G, 17, sh)) return true;
  if (b.m < 9 || b.m > 16) return false;
  // four row tiles on sixteen waves, within a launch's own K split
  if (plan6(b, G, 9, sh) && sh.rt == kG6Rt && sh.plan.split <= kSplitInLaunch) return true;
  Split5 sp;
  int cpw = 4, ranges = 1;
  bool stream = false;
  if (plan5<FMT, G>(b, sp, cpw, stream, ranges) && sp.split <= kSplitInLaunch) return false;
  return plan6(b, G, 9, sh) && sh.plan.split <= kSplitInLaunch;
}

template <int FMT, int G, int MT, int NW>
static hipError_t launch_t(const GemvBatch& b, hipStream_t st) {
  constexpr int U = Fmt<FMT, G>::GK == 16 ? 8 : (Fmt<FMT, G>::GK == 32 ? 4 : 2);
  int tiles = 0;
  for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemv_kernel<FMT, G, MT, NW, U>), dim3(tiles), dim3(NW * 64), 0, st, b);
  return hipGetLastError();
}

// waves per workgroup of the first kernel: enough groups per wave to keep
// several loads in flight
template <int FMT, int G>
static int nw_first(const GemvBatch& b) {
  const int ng = b.k / Fmt<FMT, G>::GK;
  return ng >= 8 * 16 ? 8 : (ng >= 4 * 8 ? 4 : (ng >= 2 * 4 ? 2 : 1));
}

template <int FMT, int G, int MT>
static hipError_t launch_nw(const GemvBatch& b, hipStream_t st) {
  switch (nw_first<FMT, G>(b)) {
    case 8: return launch_t<FMT, G, MT, 8>(b, st);
    case 4: return launch_t<FMT, G, MT, 4>(b, st);
    case 2: return launch_t<FMT, G, MT, 2>(b, st);
    default: return launch_t<FMT, G, MT, 1>(b, st);
  }
}


template <int FMT, int G>
static hipError_t launch_mt(const GemvBatch& b, hipStream_t st) {
  constexpr bool v2ok = !(FMT == GF_W4 && G == 16);
  if constexpr (FMT == GF_W4 && (G == 64 || G == 32)) {
    hipError_t err;
    Shape6 sh;
    if (choose6<FMT, G>(b, sh) && launch6<G>(b, sh, st, err)) return err;
  }
  if constexpr (v2ok) {
    if (b.k % F2<FMT, G>::CK == 0) {
      hipError_t err;
      if (launch5<FMT, G>(b, st, err)) return err;
    }
  }
  if constexpr (FMT == GF_W5 || FMT == GF_W6 || FMT == GF_BF16) {
    return hipErrorInvalidConfiguration;  // no launch shape (the formats have no other path)
  } else {
    if (b.m <= 16) return launch_nw<FMT, G, 1>(b, st);
    return launch_nw<FMT, G, 2>(b, st);
  }
}

// launch_mt's choice, described instead of launched
template <int FMT, int G>
static bool describe_mt(const GemvBatch& b, GemvPlanInfo& o) {
  constexpr bool v2ok = !(FMT == GF_W4 && G == 16);
  o = GemvPlanInfo{};
  const int mt = b.m <= 16 ? 1 : 2;
  if constexpr (FMT == GF_W4 && (G == 64 || G == 32)) {
    Shape6 sh;
    if (choose6<FMT, G>(b, sh)) {
      const int gtot = sh.plan.groups[0] + sh.plan.groups[1] + sh.plan.groups[2];
      o.kernel = 4;
      o.split = sh.plan.split;
      o.cps = sh.plan.cps;
      o.rt = sh.rt;
      o.workgroups = gtot * sh.plan.split;
      o.threads = (sh.rt == 2 ? G6<G, 1, 2>::NW : G6<G, 1, kG6Rt>::NW) * 64;
      if (sh.rt == 2)
        o.lds = mt == 2 ? G6<G, 2, 2>::LDS : G6<G, 1, 2>::LDS;
      else
        o.lds = mt == 2 ? G6<G, 2, kG6Rt>::LDS : G6<G, 1, kG6Rt>::LDS;
      o.ws_used = sh.plan.split > 1 ? (size_t)gtot * sh.plan.split * sh.rt * mt * 1024 : 0;
      return true;
    }
  }
  if constexpr (v2ok) {
    if (b.k % F2<FMT, G>::CK == 0) {
      Split5 sp;
      int cpw = 4;
      bool stream = false;
      int ranges = 1;
      if (plan5<FMT, G>(b, sp, cpw, stream, ranges)) {
        const int gtot = sp.groups[0] + sp.groups[1] + sp.groups[2];
        o.kernel = stream ? 3 : (ranges > 1 ? 2 : 1);
        o.split = sp.split;
        o.cps = sp.cps;
        o.cpw = cpw;
        o.wpt = sp.wpt;
        o.rt = sp.rt;
        o.workgroups = gtot * sp.split;
        o.threads = sp.rt * sp.wpt * 64;
        o.lds = lds5<FMT, G>(b, sp, stream, ranges);
        o.ws_used = sp.split > 1 ? (size_t)gtot * sp.split * sp.rt * mt * 1024 : 0;
        return true;
      }
    }
  }
  if constexpr (FMT == GF_W5 || FMT == GF_W6 || FMT == GF_BF16) {
    return false;
  } else {
    int tiles = 0;
    for (int i = 0; i < b.nmat; ++i) tiles += b.mat[i].tiles;
    o.kernel = 5;
    o.split = 1;
    o.rt = 1;
    o.workgroups = tiles;
    o.threads = nw_first<FMT, G>(b) * 64;
    return true;
  }
}

bool plan_gemv(const GemvBatch& b, int fmt, int group, GemvPlanInfo& out) {
  out = GemvPlanInfo{};
  if (b.m == 0) return true;
  switch (fmt) {
    case GF_W4:
      if (group == 64) return describe_mt<GF_W4, 64>(b, out);
      if (group == 32) return describe_mt<GF_W4, 32>(b, out);
      if (group == 16) return describe_mt<GF_W4, 16>(b, out);
      break;
    case GF_W8:
      if (group == 64) return describe_mt<GF_W8, 64>(b, out);
      if (group == 32) return describe_mt<GF_W8, 32>(b, out);
      if (group == 16) return describe_mt<GF_W8, 16>(b, out);
      break;
    case GF_SB:
      return describe_mt<GF_SB, 32>(b, out);
    case GF_F16:
      return describe_mt<GF_F16, 32>(b, out);
    case GF_W6:
      if (group == 64) return describe_mt<GF_W6, 64>(b, out);
      if (group == 32) return describe_mt<GF_W6, 32>(b, out);
      break;
    case GF_W5:
      if (group == 64) return describe_mt<GF_W5, 64>(b, out);
      if (group == 32) return describe_mt<GF_W5, 32>(b, out);
      break;
    case GF_BF16:
      return describe_mt<GF_BF16, 32>(b, out);
  }
  return false;
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
    case GF_W6:
      if (group == 64) return launch_mt<GF_W6, 64>(b, st);
      if (group == 32) return launch_mt<GF_W6, 32>(b, st);
      break;
    case GF_W5:
      if (group == 64) return launch_mt<GF_W5, 64>(b, st);
      if (group == 32) return launch_mt<GF_W5, 32>(b, st);
      break;
    case GF_BF16:
      return launch_mt<GF_BF16, 32>(b, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace rq
