// Dense W8A8 products on MFMA for prefill chunks:
//   fp8 : y[m][n] = fp16(s_x[m] * s_w[n] * sum_k e4m3(xq[m][k]) * e4m3(wq[n][k]))
//   int8: acc = sum_k xq[m][k] * wq[n][k] (exact int32), y = fp16(acc * s_x[m] * s_w[n])
// (RWKV-7 Quantization Toolkit, Key Design: FP8 weights on FP8 matrix cores
// with per-token activation scales, INT8 through int8 x int8 products;
// Architecture: FP8 + INT8 GEMM kernels with shape-aware tile configurations.)
//
// gfx950 mapping: v_mfma_f32_16x16x128_f8f6f4 (both operands OCP e4m3) and
// v_mfma_i32_16x16x64_i8.  A lane holds 32 (fp8) or 16 (int8) consecutive k
// of one row of each operand; A and B use the same lane -> k assignment, so
// every k meets its partner whatever order the instruction sums in.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace rq {

// BM x BN output tile per workgroup of 4 waves (2 x 2), each wave
// (BM/2) x (BN/2) as 16 x 16 MFMA blocks.
template <bool FP8, int BM, int BN>
__global__ void __launch_bounds__(256) gemm_w8a8_kernel(const uint8_t* __restrict__ xq,
                                                        const float* __restrict__ sx, int M,
                                                        const uint8_t* __restrict__ wq,
                                                        const float* __restrict__ sw, int N, int K,
                                                        uint16_t* __restrict__ y, int ldy,
                                                        int32_t* __restrict__ acc_out) {
  constexpr int WM = BM / 2 / 16;  // 16-row blocks per wave along m
  constexpr int WN = BN / 2 / 16;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int m0 = blockIdx.y * BM + (wave >> 1) * (BM / 2);
  const int n0 = blockIdx.x * BN + (wave & 1) * (BN / 2);

  const uint8_t* arow[WM];
  bool av[WM];
#pragma unroll
  for (int a = 0; a < WM; ++a) {
    const int m = m0 + a * 16 + r16;
    av[a] = m < M;
    arow[a] = xq + (size_t)(av[a] ? m : 0) * K;
  }
  const uint8_t* brow[WN];
  bool bv[WN];
#pragma unroll
  for (int b = 0; b < WN; ++b) {
    const int n = n0 + b * 16 + r16;
    bv[b] = n < N;
    brow[b] = wq + (size_t)(bv[b] ? n : 0) * K;
  }

  typedef typename std::conditional<FP8, float4v, int4v>::type AccT;
  AccT acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) acc[a][b] = AccT{0, 0, 0, 0};

  for (int k0 = 0; k0 < K; k0 += 128) {
    if (FP8) {
      int8v fa[WM], fb[WN];
#pragma unroll
      for (int a = 0; a < WM; ++a) {
        const uint4* p = (const uint4*)(arow[a] + k0 + 32 * q);
        uint4 lo = av[a] ? p[0] : make_uint4(0, 0, 0, 0);
        uint4 hi = av[a] ? p[1] : make_uint4(0, 0, 0, 0);
        fa[a] = int8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int b = 0; b < WN; ++b) {
        const uint4* p = (const uint4*)(brow[b] + k0 + 32 * q);
        uint4 lo = bv[b] ? p[0] : make_uint4(0, 0, 0, 0);
        uint4 hi = bv[b] ? p[1] : make_uint4(0, 0, 0, 0);
        fb[b] = int8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0, 0,
                                                                       0, 0, 0);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int4v fa[WM], fb[WN];
#pragma unroll
        for (int a = 0; a < WM; ++a) {
          uint4 v = av[a] ? *(const uint4*)(arow[a] + k0 + 64 * h + 16 * q) : make_uint4(0, 0, 0, 0);
          fa[a] = int4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int b = 0; b < WN; ++b) {
          uint4 v = bv[b] ? *(const uint4*)(brow[b] + k0 + 64 * h + 16 * q) : make_uint4(0, 0, 0, 0);
          fb[b] = int4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int a = 0; a < WM; ++a)
#pragma unroll
          for (int b = 0; b < WN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds D[m = 4q + r][n = r16] of each 16 x 16 block
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const int n = n0 + b * 16 + r16;
      if (n >= N) continue;
      const float swn = sw[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + a * 16 + 4 * q + r;
        if (m >= M) continue;
        const float v = FP8 ? (float)acc[a][b][r] : (float)acc[a][b][r];
        if (acc_out) acc_out[(size_t)m * N + n] = (int32_t)acc[a][b][r];
        if (y) y[(size_t)m * ldy + n] = f32_to_f16_bits(v * sx[m] * swn);
      }
    }
}

hipError_t launch_gemm_w8a8(const void* xq, const float* sx, int m, const void* wq, const float* sw,
                            int n, int k, bool fp8, uint16_t* y, int ldy, int32_t* acc_out,
                            hipStream_t st) {
  if (m == 0 || n == 0) return hipSuccess;
  constexpr int BM = 64, BN = 64;
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  if (fp8)
    hipLaunchKernelGGL((gemm_w8a8_kernel<true, BM, BN>), grid, dim3(256), 0, st, (const uint8_t*)xq, sx, m,
                       (const uint8_t*)wq, sw, n, k, y, ldy, acc_out);
  else
    hipLaunchKernelGGL((gemm_w8a8_kernel<false, BM, BN>), grid, dim3(256), 0, st, (const uint8_t*)xq, sx,
                       m, (const uint8_t*)wq, sw, n, k, y, ldy, acc_out);
  return hipGetLastError();
}

}  // namespace rq
