// Prefill products on int4 codes, any number of activation rows (the prefill
// chunks of 64 to 1024 tokens):
//   y[m][n] = fp16( sum_k x[m][k] * w[n][k] ),  accumulated in fp32, with
//   w = fp16(q * s) on symmetric int4 group codes (groups of 16, 32 or 64);
//   on asymmetric 256-superblocks, per 32-group j,
//   sum_k x w = S_j * sum_k x u - M_j * sum_k x, the two sums on MFMA (codes
//   u are exact fp16 integers) and S_j, M_j applied in fp32.
// This is the tensor-core GEMM member of the int4 product family ("RWKV-7 G1
// 1.5B -- int4 GPTQ for rwkv-sglang" model card, summary), here on gfx950
// MFMA; the weights are read as codes and dequantized in registers, never
// written out.  Beyond fp32 summation: symmetric, q * s is rounded once to
// fp16 (q has 3 significant bits, s 11), at most 2^-11 of each weight (one
// fp16 rounding); superblocks, nothing is rounded below fp32 (the B operands
// sc_j u and mc_j are exact fp16 integers, the products exact; the MFMA sums
// over a 128-k block and its scalings by d and dmin round in fp32).
//
// A workgroup of NW waves (4 or 8) computes a BM x BN output tile; the waves
// form a WM x (NW / WM) grid and each computes its (BM / WM) x (BN WM / NW)
// part as 16 x 16 v_mfma_f32_16x16x32_f16 tiles over the workgroup's k
// blocks.  With WM = 1 no two waves decode the same codes.  K runs in blocks
// of 128.  For each block the x rows (BM x 256 bytes, whole 128-byte lines)
// and the code rows (BN x 64 bytes) are copied by LDS DMA into a 3-stage ring
// shared by the workgroup, so two blocks are in flight while one is
// multiplied; one barrier per block.  The x segments of a row are stored at
// slot segment ^ (row % 16) and the code segments at
// segment ^ ((row / 4) % 4), so the 16 rows a fragment read touches fall in
// distinct LDS banks.  Split along K (part != null), workgroup z of gridDim.z
// takes k blocks [z kbs, (z + 1) kbs) and stores its fp32 tile to
// part[z][m][n]; gemm_w4_reduce_kernel adds the slices in order.
//
// k mapping: lane l (row l % 16 of a tile, quarter q = l / 16) reads one
// 16-byte code segment per n tile and block, segment q of the row's 64 bytes.
// Its four words are the B operands of the block's four MFMA k steps: word s
// holds k = 32 q + 8 s + 0..7, decoded to exact fp16 integers by dec4n and
// scaled in packed fp16 by that group's scale.  The A operand of step s is
// the 16 bytes of x holding the same eight k, so every product pairs matching
// k whatever order the MFMA sums in.  The block's scales (64 / G dwords per
// row; for superblocks d, dmin and the 12 sub-code bytes of the block's
// superblock) are copied into the same ring stage by LDS DMA.
//
// Every copy and its wait are inline asm: the compiler cannot tell which LDS
// bytes a DMA writes and would otherwise wait for every load in flight before
// each LDS read, and a plain load into registers among the copies would make
// its own wait drain them all.  The DMA writes no register, and every LDS read
// of its bytes follows an explicit wait and a barrier.  Rows past m (n) read
// row m - 1 (n - 1) and only reach outputs that are never stored.
#include "device_common.h"
#include "kernels.h"

namespace rq {

// lane exchanges (v_permlane32_swap / v_permlane16_swap) for the word transpose
__device__ __forceinline__ void swap32w(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16w(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

template <bool SB, int G, int BM, int BN, int WM, int NW>
__global__ void __launch_bounds__(64 * NW) gemm_w4_kernel(const W4Gemm p, int kbs, float* __restrict__ part) {
  constexpr int WN = NW / WM;
  constexpr int TM = BM / (16 * WM), TN = BN / (16 * WN);  // 16 x 16 tiles of a wave in m and n
  constexpr int D = SB ? 1 : 64 / G;          // symmetric: scale dwords per row and block
  // scale area per stage: symmetric, D dwords per row; superblocks, d and dmin
  // in a 4-byte slot each and the 12 sub-code bytes in a 16-byte slot per row
  constexpr int SS = SB ? BN * 24 : BN * 4 * D;
  constexpr int SX = BM * 256, SC = BN * 64, STAGE = SX + SC + SS;
  constexpr int NB = 3;
  constexpr int XPW = BM / (4 * NW);          // x DMA instructions per wave per block
  constexpr int CPW = BN / (16 * NW);         // code DMA instructions per wave per block
  static_assert(XPW * 4 * NW == BM && CPW * 16 * NW == BN && TM >= 1 && TN >= 1, "tile splits evenly");
  constexpr int SDW = BN * D / NW;            // symmetric: scale dwords per wave per block
  constexpr int RPW = BN / NW;                // superblocks: rows per wave
  static_assert(!SB || RPW <= 64, "one superblock copy per wave and kind");
  constexpr int SPW = SB ? 3 : (SDW + 63) / 64;  // scale DMA instructions per wave per block
  constexpr int OPS = XPW + CPW + SPW;        // vector memory instructions per wave per block
  extern __shared__ uint4 lds4[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int M = p.m, N = p.n, K = p.k;
  const int kb0 = blockIdx.z * kbs;
  const int nkb = min(K >> 7, kb0 + kbs) - kb0;  // this workgroup's k blocks

  // DMA sources.  x instruction g (0 .. BM/4 - 1) copies rows 4g .. 4g + 3:
  // lane -> row 4g + lane / 16, slot lane % 16.  Code instruction g
  // (0 .. BN/16 - 1) copies rows 16g .. 16g + 15: lane -> row 16g + lane / 4,
  // slot lane % 4.  Scale dword t (0 .. BN D - 1) is dword t % D of row t / D.
  const uint16_t* xsrc[XPW];
  const uint8_t* csrc[CPW];
  const uint8_t* ssrc[SPW];
  bool sact[SPW];
#pragma unroll
  for (int u = 0; u < XPW; ++u) {
    const int r = 4 * (wave * XPW + u) + (lane >> 4);
    const int seg = (lane & 15) ^ (r & 15);
    xsrc[u] = p.x + (size_t)min(m0 + r, M - 1) * p.ldx + (size_t)kb0 * 128 + seg * 8;
  }
  const size_t crow = (size_t)(K >> 1);
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int r = 16 * (wave * CPW + u) + (lane >> 2);
    const int seg = (lane & 3) ^ ((r >> 2) & 3);
    csrc[u] = p.codes + (size_t)min(n0 + r, N - 1) * crow + (size_t)kb0 * 64 + seg * 16;
  }
  if constexpr (SB) {
    // lane -> row wave * RPW + lane: d, dmin (2 bytes each) and sub (12 bytes)
    // of the row's superblock; the block's superblock is added per copy
    const size_t nsb = (size_t)(K / 256);
    const size_t rsb = (size_t)min(n0 + wave * RPW + lane, N - 1) * nsb;
#pragma unroll
    for (int u = 0; u < 3; ++u) sact[u] = lane < RPW;
    ssrc[0] = (const uint8_t*)p.scales + rsb * 2;
    ssrc[1] = (const uint8_t*)p.mins + rsb * 2;
    ssrc[2] = p.sub + rsb * 12;
  } else {
    const size_t srow = (size_t)(K / G) * 2;  // scale bytes per row
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int i = u * 64 + lane;           // dword of this wave's share
      const int t = wave * SDW + i;
      sact[u] = i < SDW;
      ssrc[u] = (const uint8_t*)p.scales + (size_t)min(n0 + t / D, N - 1) * srow + (size_t)kb0 * (4 * D) +
                (t % D) * 4;
    }
  }
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;

  auto issue = [&](int kb, int st) {
    const uint32_t base = ring + st * STAGE;
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
      const uint16_t* g = xsrc[u] + (size_t)kb * 128;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(base + (wave * XPW + u) * 1024) : "memory", "m0");
    }
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const uint8_t* g = csrc[u] + (size_t)kb * 64;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(base + SX + (wave * CPW + u) * 1024) : "memory", "m0");
    }
    if constexpr (SB) {
      // 2-byte copies land zero-extended in 4-byte slots, 12-byte copies in
      // 16-byte slots (one per lane)
      const size_t sb = (size_t)((kb0 + kb) >> 1);
      if (sact[0]) {
        const uint8_t* gd = ssrc[0] + sb * 2;
        const uint8_t* gm = ssrc[1] + sb * 2;
        const uint8_t* gs = ssrc[2] + sb * 12;
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
                     :: "v"(gd), "s"(base + SX + SC + wave * RPW * 4) : "memory", "m0");
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
                     :: "v"(gm), "s"(base + SX + SC + BN * 4 + wave * RPW * 4) : "memory", "m0");
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %0, off"
                     :: "v"(gs), "s"(base + SX + SC + BN * 8 + wave * RPW * 16) : "memory", "m0");
      }
    } else {
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        const uint8_t* g = ssrc[u] + (size_t)kb * (4 * D);
        if (sact[u])
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                       :: "v"(g), "s"(base + SX + SC + (wave * SDW + u * 64) * 4) : "memory", "m0");
      }
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int j, int st) {
    const uint8_t* xs = (const uint8_t*)lds4 + st * STAGE;
    const uint8_t* cs = xs + SX;
    const uint8_t* ss = xs + SX + SC;
    if constexpr (SB) {
      // superblocks: a 4 x 4 word transpose across the lane quarters gives
      // lane q word q of each of the block's four 32-groups, so k step s
      // covers group s alone.  With S_s = d sc_s and M_s = dmin mc_s, the
      // block's sum is d sum_s sum_k x (sc_s u) - dmin sum_s sum_k x mc_s: the
      // B operands sc_s u (at most 63 * 15) and mc_s are exact fp16 integers,
      // so two MFMA chains per tile accumulate the block exactly up to fp32
      // summation, and d and dmin are applied once per block in fp32
      uint32_t wv[TN][4];
      uint32_t scc[TN][4], mcc[TN][4];  // the 6-bit codes, as fp16 bits (exact)
      float dd[TN], dmm[TN];
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int row = wn * (BN / WN) + 16 * b + r16;
        const uint4 c4 = *(const uint4*)(cs + row * 64 + ((q ^ ((row >> 2) & 3)) << 4));
        uint32_t w0 = c4.x, w1 = c4.y, w2 = c4.z, w3 = c4.w;
        swap32w(w0, w2);
        swap32w(w1, w3);
        swap16w(w0, w1);
        swap16w(w2, w3);
        wv[b][0] = w0;
        wv[b][1] = w1;
        wv[b][2] = w2;
        wv[b][3] = w3;
        dd[b] = f16_bits_to_f32(*(const uint16_t*)(ss + row * 4));
        dmm[b] = f16_bits_to_f32(*(const uint16_t*)(ss + BN * 4 + row * 4));
        const uint4 sub = *(const uint4*)(ss + BN * 8 + row * 16);
        const uint64_t lo48 = (uint64_t)sub.x | ((uint64_t)(sub.y & 0xffffu) << 32);
        const uint64_t hi48 = (uint64_t)(sub.y >> 16) | ((uint64_t)sub.z << 16);
        const int g0 = ((kb0 + j) & 1) * 4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // an integer c < 64 is fp16 (1024 + c) - 1024: the bias trick of dec4n
          const uint32_t c1 = (uint32_t)(lo48 >> (6 * (g0 + s))) & 63u;
          const uint32_t c2 = (uint32_t)(hi48 >> (6 * (g0 + s))) & 63u;
          scc[b][s] = hsub2(0x64006400u | c1 | (c1 << 16), 0x64006400u);
          mcc[b][s] = hsub2(0x64006400u | c2 | (c2 << 16), 0x64006400u);
        }
      }
      float4v r[TM][TN], rm[TM][TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          r[a][b] = float4v{0.f, 0.f, 0.f, 0.f};
          rm[a][b] = float4v{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8 bf[TN], bm[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          // sc_s u: packed fp16 products of integers below 2^11, exact
          const uint4 u = __builtin_bit_cast(uint4, dec4n<false>(wv[b][s]));
          const half2v c = __builtin_bit_cast(half2v, scc[b][s]);
          bf[b] = __builtin_bit_cast(half8, make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u.x) * c),
                                                       __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u.y) * c),
                                                       __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u.z) * c),
                                                       __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u.w) * c)));
          bm[b] = __builtin_bit_cast(half8, make_uint4(mcc[b][s], mcc[b][s], mcc[b][s], mcc[b][s]));
        }
#pragma unroll
        for (int a = 0; a < TM; ++a) {
          const int row = wm * (BM / WM) + 16 * a + r16;
          const half8 af = *(const half8*)(xs + row * 256 + (((4 * s + q) ^ (row & 15)) << 4));
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            r[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b], r[a][b], 0, 0, 0);
            rm[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bm[b], rm[a][b], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][b][i] += dd[b] * r[a][b][i] - dmm[b] * rm[a][b][i];
      return;
    }
    uint4 cw[TN];
    half8 s01[TN], s23[TN];  // the lane's scale for steps 0-1 and 2-3, broadcast
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int row = wn * (BN / WN) + 16 * b + r16;
      cw[b] = *(const uint4*)(cs + row * 64 + ((q ^ ((row >> 2) & 3)) << 4));
      // group of k = 32 q + 8 s within the block: g64 -> q / 2, g32 -> q, g16 -> 2 q + s / 2
      _Float16 lo, hi;
      if constexpr (G == 16) {
        const half2v v = *(const half2v*)(ss + row * 16 + q * 4);
        lo = v[0];
        hi = v[1];
      } else {
        lo = *(const _Float16*)(ss + row * 4 * D + (G == 64 ? (q >> 1) : q) * 2);
        hi = lo;
      }
      s01[b] = half8{lo, lo, lo, lo, lo, lo, lo, lo};
      s23[b] = half8{hi, hi, hi, hi, hi, hi, hi, hi};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 bf[TN];
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const uint32_t w = s == 0 ? cw[b].x : (s == 1 ? cw[b].y : (s == 2 ? cw[b].z : cw[b].w));
        bf[b] = dec4n<true>(w) * (s < 2 ? s01[b] : s23[b]);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int row = wm * (BM / WM) + 16 * a + r16;
        const half8 af = *(const half8*)(xs + row * 256 + (((4 * q + s) ^ (row & 15)) << 4));
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b], acc[a][b], 0, 0, 0);
      }
    }
  };

  // block j lives in stage j % 3; after the wait and barrier of iteration j
  // every wave's copies of block j have landed and every wave is done with
  // block j - 1, whose stage then receives block j + 2
  if (nkb > 0) issue(0, 0);
  if (nkb > 1) issue(1, 1);
  for (int j = 0; j < nkb; ++j) {
    if (j + 1 < nkb)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(OPS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < nkb) issue(j + 2, (j + 2) % NB);
    compute(j, j % NB);
  }

  // epilogue: lane holds D[m = 4q + r][n = r16] of each 16 x 16 tile
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = n0 + wn * (BN / WN) + 16 * b + r16;
    if (n >= N) continue;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / WM) + 16 * a + 4 * q + r;
        if (m >= M) continue;
        if (part)
          part[((size_t)blockIdx.z * M + m) * N + n] = acc[a][b][r];
        else
          p.y[(size_t)m * p.ldy + n] = f32_to_f16_bits(acc[a][b][r]);
      }
  }
}

// Split K, second step: y = fp16 of the slices' fp32 tiles added in slice
// order, one thread per output; every slice's load is issued before the
// first add (split <= 16).
__global__ void __launch_bounds__(256) gemm_w4_reduce_kernel(const float* __restrict__ part, int split,
                                                             const W4Gemm p) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t mn = (size_t)p.m * p.n;
  if (i >= mn) return;
  const int m = (int)(i / p.n), n = (int)(i - (size_t)m * p.n);
  float vals[16];
#pragma unroll
  for (int z = 0; z < 16; ++z) vals[z] = z < split ? part[(size_t)z * mn + i] : 0.f;
  float v = vals[0];
#pragma unroll
  for (int z = 1; z < 16; ++z)
    if (z < split) v += vals[z];
  p.y[(size_t)m * p.ldy + n] = f32_to_f16_bits(v);
}

template <bool SB, int G, int BM, int BN, int WM, int NW>
static hipError_t launch_w4_t(const W4Gemm& p, int split, float* part, hipStream_t st) {
  constexpr size_t lds = (size_t)3 * (BM * 256 + BN * 64 + (SB ? BN * 24 : BN * 256 / G));
  static_assert(lds <= 160 * 1024, "ring fits LDS");
  static const bool attr_set = hipFuncSetAttribute((const void*)gemm_w4_kernel<SB, G, BM, BN, WM, NW>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds) == hipSuccess;
  (void)attr_set;
  const int nkb = p.k >> 7;
  const int kbs = (nkb + split - 1) / split;
  const dim3 grid((unsigned)((p.n + BN - 1) / BN), (unsigned)((p.m + BM - 1) / BM), (unsigned)split);
  hipLaunchKernelGGL((gemm_w4_kernel<SB, G, BM, BN, WM, NW>), grid, dim3(64 * NW), lds, st, p, kbs,
                     split > 1 ? part : nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || split == 1) return err;
  const size_t outs = (size_t)p.m * p.n;
  hipLaunchKernelGGL(gemm_w4_reduce_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, split, p);
  return hipGetLastError();
}

// Launch plan, from measurements of the width-4096 shapes at m = 64, 256 and
// 1024 (activation + code traffic per output is K (2 / BN + 1 / (2 BM))
// bytes; eight waves let one wave's decoding overlap another's MFMAs).
// Tiles in order: 128 x 256 and 128 x 128 with eight waves (2 x 4), 64 x 256
// with four (1 x 4), 64 x 128 with eight (1 x 8), 64 x 64 with four (2 x 2);
// 128-row tiles only for m > 64, and no 128 x 256 for superblocks (its ring
// would not fit LDS).  Up to 32 k blocks (K <= 4096),
// the first tile that makes 256 workgroups unsplit; otherwise, and for longer
// K, the first that makes 256 with K split in 2, 4 or 8 slices of at least 8
// k blocks (partial tiles in the workspace); failing both, 64 x 64 split as
// far as that allows.
struct W4Plan {
  int bm, bn, wm, split, nw;
};

static W4Plan plan_w4(const W4Gemm& p, bool sb, size_t ws_bytes) {
  static const W4Plan tiles[] = {{128, 256, 2, 1, 8}, {128, 128, 2, 1, 8}, {64, 256, 1, 1, 4}, {64, 128, 1, 1, 8},
                                 {64, 64, 2, 1, 4}};
  const int nkb = p.k >> 7;
  auto wgs = [&](const W4Plan& t) { return (long)((p.m + t.bm - 1) / t.bm) * (long)((p.n + t.bn - 1) / t.bn); };
  auto split_ok = [&](int split) {
    return nkb / split >= 8 && (size_t)split * p.m * p.n * 4 <= ws_bytes;
  };
  // 128-row tiles only for m > 64; superblocks' ring of 128 x 256 exceeds LDS
  auto usable = [&](const W4Plan& t) { return !(t.bm == 128 && p.m <= 64) && !(sb && t.bm == 128 && t.bn == 256); };
  if (nkb <= 32)
    for (const W4Plan& t : tiles)
      if (usable(t) && wgs(t) >= 256) return t;
  for (const W4Plan& t : tiles) {
    if (!usable(t)) continue;
    for (int split = 2; split <= 8; split *= 2)
      if (split_ok(split) && wgs(t) * split >= 256) return W4Plan{t.bm, t.bn, t.wm, split, t.nw};
  }
  int split = 1;
  while (split < 8 && split_ok(2 * split) && wgs(tiles[4]) * split < 256) split *= 2;
  return W4Plan{64, 64, 2, split, 4};
}

template <bool SB, int G>
static hipError_t launch_w4_g(const W4Gemm& p, const W4Plan& pl, float* ws, hipStream_t st) {
#define RQ_W4(BM, BN, WM, NW)                                                  \
  if (pl.bm == BM && pl.bn == BN && pl.wm == WM && pl.nw == NW)                 \
    return launch_w4_t<SB, G, BM, BN, WM, NW>(p, pl.split, ws, st);
  if constexpr (!SB) {
    RQ_W4(128, 256, 2, 8)
  }
  RQ_W4(128, 128, 2, 8)
  RQ_W4(64, 256, 1, 4)
  RQ_W4(64, 128, 1, 8)
#undef RQ_W4
  return launch_w4_t<SB, G, 64, 64, 2, 4>(p, pl.split, ws, st);
}

hipError_t launch_gemm_w4(const W4Gemm& p, bool sb, int group, float* ws, size_t ws_bytes, hipStream_t st) {
  if (p.m == 0 || p.n == 0) return hipSuccess;
  const W4Plan pl = plan_w4(p, sb, ws ? ws_bytes : 0);
  if (sb) return launch_w4_g<true, 32>(p, pl, ws, st);
  if (group == 64) return launch_w4_g<false, 64>(p, pl, ws, st);
  if (group == 32) return launch_w4_g<false, 32>(p, pl, ws, st);
  if (group == 16) return launch_w4_g<false, 16>(p, pl, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace rq
