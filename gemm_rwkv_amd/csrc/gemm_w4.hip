// Prefill products on int4 codes, any number of activation rows (the prefill
// chunks of 64 to 1024 tokens):
//   y[m][n] = fp16( sum_k x[m][k] * w[n][k] ),  w = fp16(q * s),
// on symmetric int4 group codes (groups of 16, 32 or 64), accumulated in fp32.
// This is the tensor-core GEMM member of the int4 product family ("RWKV-7 G1
// 1.5B -- int4 GPTQ for rwkv-sglang" model card, summary), here on gfx950
// MFMA; the weights are read as codes and dequantized in registers, never
// written out.  The one rounding beyond fp32 summation is that of q * s to
// fp16 (q has 3 significant bits, s 11), at most 2^-12 of each weight.
//
// A workgroup of four waves computes a BM x BN output tile (BM, BN in
// {64, 128}); each wave computes a (BM / 2) x (BN / 2) quarter as 16 x 16
// v_mfma_f32_16x16x32_f16 tiles over all of K.  K runs in blocks of 128.  For
// each block the x rows (BM x 256 bytes, whole 128-byte lines) and the code
// rows (BN x 64 bytes) are copied by LDS DMA into a 3-stage ring shared by
// the workgroup, so two blocks are in flight while one is multiplied; one
// barrier per block.  The x segments of a row are stored at slot
// segment ^ (row % 16) and the code segments at segment ^ ((row / 4) % 4), so
// the 16 rows a fragment read touches fall in distinct LDS banks.
//
// k mapping: lane l (row l % 16 of a tile, quarter q = l / 16) reads one
// 16-byte code segment per n tile and block, segment q of the row's 64 bytes.
// Its four words are the B operands of the block's four MFMA k steps: word s
// holds k = 32 q + 8 s + 0..7, decoded to exact fp16 integers by dec4n and
// scaled in packed fp16 by that group's scale.  The A operand of step s is
// the 16 bytes of x holding the same eight k, so every product pairs matching
// k whatever order the MFMA sums in.  The block's scales (64 / G dwords per
// row) are copied into the same ring stage by LDS DMA.
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

template <int G, int BM, int BN>
__global__ void __launch_bounds__(256) gemm_w4_kernel(const W4Gemm p) {
  constexpr int TM = BM / 32, TN = BN / 32;   // 16 x 16 tiles of a wave in m and n
  constexpr int D = 64 / G;                   // scale dwords per row and block
  constexpr int SX = BM * 256, SC = BN * 64, SS = BN * 4 * D, STAGE = SX + SC + SS;
  constexpr int NB = 3;
  constexpr int XPW = BM / 16;                // x DMA instructions per wave per block
  constexpr int CPW = BN / 64;                // code DMA instructions per wave per block
  constexpr int SDW = BN * D / 4;             // scale dwords per wave per block
  constexpr int SPW = (SDW + 63) / 64;        // scale DMA instructions per wave per block
  constexpr int OPS = XPW + CPW + SPW;        // vector memory instructions per wave per block
  extern __shared__ uint4 lds4[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int M = p.m, N = p.n, K = p.k;
  const int nkb = K >> 7;

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
    xsrc[u] = p.x + (size_t)min(m0 + r, M - 1) * p.ldx + seg * 8;
  }
  const size_t crow = (size_t)(K >> 1);
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int r = 16 * (wave * CPW + u) + (lane >> 2);
    const int seg = (lane & 3) ^ ((r >> 2) & 3);
    csrc[u] = p.codes + (size_t)min(n0 + r, N - 1) * crow + seg * 16;
  }
  const size_t srow = (size_t)(K / G) * 2;  // scale bytes per row
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int i = u * 64 + lane;             // dword of this wave's share
    const int t = wave * SDW + i;
    sact[u] = i < SDW;
    ssrc[u] = (const uint8_t*)p.scales + (size_t)min(n0 + t / D, N - 1) * srow + (t % D) * 4;
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
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const uint8_t* g = ssrc[u] + (size_t)kb * (4 * D);
      if (sact[u])
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     :: "v"(g), "s"(base + SX + SC + (wave * SDW + u * 64) * 4) : "memory", "m0");
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st) {
    const uint8_t* xs = (const uint8_t*)lds4 + st * STAGE;
    const uint8_t* cs = xs + SX;
    const uint8_t* ss = xs + SX + SC;
    uint4 cw[TN];
    half8 s01[TN], s23[TN];  // the lane's scale for steps 0-1 and 2-3, broadcast
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int row = wn * (BN / 2) + 16 * b + r16;
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
        const int row = wm * (BM / 2) + 16 * a + r16;
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
    compute(j % NB);
  }

  // epilogue: lane holds D[m = 4q + r][n = r16] of each 16 x 16 tile
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = n0 + wn * (BN / 2) + 16 * b + r16;
    if (n >= N) continue;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / 2) + 16 * a + 4 * q + r;
        if (m < M) p.y[(size_t)m * p.ldy + n] = f32_to_f16_bits(acc[a][b][r]);
      }
  }
}

template <int G, int BM, int BN>
static hipError_t launch_w4_t(const W4Gemm& p, hipStream_t st) {
  constexpr size_t lds = (size_t)3 * (BM * 256 + BN * 64 + BN * 256 / G);
  static const bool attr_set = hipFuncSetAttribute((const void*)gemm_w4_kernel<G, BM, BN>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds) == hipSuccess;
  (void)attr_set;
  const dim3 grid((unsigned)((p.n + BN - 1) / BN), (unsigned)((p.m + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_w4_kernel<G, BM, BN>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

// Tile: 128 x 128 when m > 64 and that gives one workgroup per compute unit
// (256), else 64 x 128 when that does, else 64 x 64.
template <int G>
static hipError_t launch_w4_g(const W4Gemm& p, hipStream_t st) {
  const long mt128 = (p.m + 127) / 128, mt64 = (p.m + 63) / 64;
  const long nt128 = (p.n + 127) / 128;
  if (p.m > 64 && mt128 * nt128 >= 256) return launch_w4_t<G, 128, 128>(p, st);
  if (mt64 * nt128 >= 256) return launch_w4_t<G, 64, 128>(p, st);
  return launch_w4_t<G, 64, 64>(p, st);
}

hipError_t launch_gemm_w4(const W4Gemm& p, int group, hipStream_t st) {
  if (p.m == 0 || p.n == 0) return hipSuccess;
  if (group == 64) return launch_w4_g<64>(p, st);
  if (group == 32) return launch_w4_g<32>(p, st);
  if (group == 16) return launch_w4_g<16>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace rq
