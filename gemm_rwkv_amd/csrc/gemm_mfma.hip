// Dense W8A8 products on MFMA for prefill chunks:
//   fp8 : y[m][n] = fp16(s_x[m] * s_w[n] * sum_k e4m3(xq[m][k]) * e4m3(wq[n][k]))
//   int8: acc = sum_k xq[m][k] * wq[n][k] (exact int32), y = fp16(acc * s_x[m] * s_w[n])
// (RWKV-7 Quantization Toolkit, Key Design: FP8 weights on FP8 matrix cores
// with per-token activation scales, INT8 through int8 x int8 products;
// Architecture: FP8 + INT8 GEMM kernels with shape-aware tile configurations.)
//
// gfx950 mapping: v_mfma_f32_16x16x128_f8f6f4 (both operands OCP e4m3) and
// v_mfma_i32_16x16x64_i8.  A lane holds 32 (fp8) or 16 (int8) k of one row of
// each operand; x and w use the same lane -> k assignment, so every k meets
// its partner whatever order the instruction sums in.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace rq {

// One workgroup computes a (16 TM) x (16 TN) output tile.  Its KW waves
// split K (wave w takes the 128-wide k blocks w, w + KW, ...) and each covers
// the whole tile, so no operand byte is read twice within a workgroup; the
// KW partial tiles are summed through LDS in wave order (deterministic),
// scaled and stored.
//
// Operands reach the MFMA layout through LDS.  A lane's operand is 32 bytes
// of one row (row = lane % 16), so loading straight into registers makes each
// instruction touch 16 rows x 64 B, half of every 128-byte line, which
// halves what L2 delivers per instruction.  Instead each wave copies its k
// block with LDS DMA reads of 8 rows x 128 B (whole lines) into a private
// 2-stage ring and reads the fragments back with ds_read_b128.  The 16-byte
// segments of row r are stored at slot (segment ^ (r % 8)), and lane
// (row r16 = lane % 16, q = lane / 16) takes segments q and q + 4 of its row
// (32 bytes, the same k for x and w, so every k still meets its partner):
// then the sixteen lanes that LDS serves together read sixteen distinct
// 16-byte bank groups.  (Segments 2q and 2q + 1 under the swizzle
// (r / 2) % 8 cost four bank-conflict cycles per read, counted with
// SQ_LDS_BANK_CONFLICT.)  While block j is multiplied, block j + 1 is in
// flight.
//
// The DMA and its waits are issued as inline asm: the compiler cannot tell
// which LDS bytes an LDS DMA writes, and would otherwise wait for every DMA
// in flight before any LDS read.  The DMA writes no register, and every read
// of its LDS bytes comes after an explicit wait with a memory clobber.
//
// Rows past m (n) read row m - 1 (n - 1): they only reach outputs that are
// never stored.  fp8: a lane's 32 bytes are one operand of v_mfma 16x16x128
// f8f6f4; int8: each 16-byte half feeds one v_mfma_i32_16x16x64_i8.
template <bool FP8, int TM, int TN, int KW>
__global__ void __launch_bounds__(64 * KW) gemm_w8a8_kernel(const uint8_t* __restrict__ xq,
                                                            const float* __restrict__ sx, int M,
                                                            const uint8_t* __restrict__ wq,
                                                            const float* __restrict__ sw, int N, int K,
                                                            uint16_t* __restrict__ y, int ldy,
                                                            int32_t* __restrict__ acc_out) {
  constexpr int BM = 16 * TM, BN = 16 * TN;
  constexpr int SA = BM * 128, STAGE = (BM + BN) * 128;  // bytes of one staged k block
  constexpr int NB = 2;                                   // stages per wave
  typedef typename std::conditional<FP8, float4v, int4v>::type AccT;
  extern __shared__ uint4 lds4[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int nkb = K >> 7;

  // LDS DMA sources: instruction i covers tile rows 8i .. 8i + 7, lane ->
  // row 8i + lane / 8, LDS slot lane % 8 holding segment slot ^ (row % 8)
  const int drow = lane >> 3, dslot = lane & 7;
  const uint8_t* asrc[TM * 2];
  const uint8_t* bsrc[TN * 2];
#pragma unroll
  for (int i = 0; i < TM * 2; ++i) {
    const int r = 8 * i + drow;
    asrc[i] = xq + (size_t)min(m0 + r, M - 1) * K + ((dslot ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < TN * 2; ++i) {
    const int r = 8 * i + drow;
    bsrc[i] = wq + (size_t)min(n0 + r, N - 1) * K + ((dslot ^ (r & 7)) << 4);
  }
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4 + wave * NB * STAGE;
  auto dma = [&](int st, int kb) {
    const uint32_t base = ring + st * STAGE;
#pragma unroll
    for (int i = 0; i < TM * 2; ++i) {
      const uint8_t* g = asrc[i] + (size_t)kb * 128;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(base + i * 1024) : "memory", "m0");
    }
#pragma unroll
    for (int i = 0; i < TN * 2; ++i) {
      const uint8_t* g = bsrc[i] + (size_t)kb * 128;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(base + SA + i * 1024) : "memory", "m0");
    }
  };

  // fragment reads: row r16 of a 16-row block, segments q and q + 4
  const int swz = r16 & 7;
  const int o0 = r16 * 128 + ((q ^ swz) << 4);
  const int o1 = r16 * 128 + (((q + 4) ^ swz) << 4);
  const uint8_t* my = (const uint8_t*)lds4 + wave * NB * STAGE;

  AccT acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = AccT{0, 0, 0, 0};

  auto compute = [&](int st) {
    const uint8_t* base = my + st * STAGE;
    uint4 fa[TM][2], fb[TN][2];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      fa[a][0] = *(const uint4*)(base + a * 2048 + o0);
      fa[a][1] = *(const uint4*)(base + a * 2048 + o1);
    }
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      fb[b][0] = *(const uint4*)(base + SA + b * 2048 + o0);
      fb[b][1] = *(const uint4*)(base + SA + b * 2048 + o1);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const uint4 al = fa[a][0], ah = fa[a][1];
        const uint4 bl = fb[b][0], bh = fb[b][1];
        if constexpr (FP8) {
          const int8v av = {(int)al.x, (int)al.y, (int)al.z, (int)al.w, (int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int8v bv = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w, (int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[a][b], 0, 0, 0, 0, 0, 0);
        } else {
          const int4v a0 = {(int)al.x, (int)al.y, (int)al.z, (int)al.w};
          const int4v b0 = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w};
          const int4v a1 = {(int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int4v b1 = {(int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[a][b], 0, 0, 0);
        }
      }
  };

  // this wave's blocks j = 0 .. nmine - 1 are k blocks wave + j KW; block j
  // lives in stage j % 2 and block j + 1 is in flight while j is multiplied
  constexpr int PER = (TM + TN) * 2;  // DMA instructions per block
  const int nmine = nkb > wave ? (nkb - wave + KW - 1) / KW : 0;
  if (nmine > 0) dma(0, wave);
  for (int j = 0; j < nmine; ++j) {
    if (j + 1 < nmine) {
      dma((j + 1) & 1, wave + (j + 1) * KW);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER) : "memory");  // block j has landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    compute(j & 1);
  }

  // epilogue, one block row at a time, in the (now free) staging area: lane
  // holds D[m = 4q + r][n = r16] of each 16 x 16 block
  AccT (*red)[TN][64] = (AccT (*)[TN][64])lds4;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
    __syncthreads();  // staging reads, or the previous row's sums, are done
#pragma unroll
    for (int b = 0; b < TN; ++b) red[wave][b][lane] = acc[a][b];
    __syncthreads();
    for (int b = wave; b < TN; b += KW) {
      AccT v = red[0][b][lane];
#pragma unroll
      for (int w = 1; w < KW; ++w) {
        const AccT u = red[w][b][lane];
        v[0] += u[0];
        v[1] += u[1];
        v[2] += u[2];
        v[3] += u[3];
      }
      const int n = n0 + b * 16 + r16;
      if (n >= N) continue;
      const float swn = y ? sw[n] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + a * 16 + 4 * q + r;
        if (m >= M) continue;
        if (acc_out) acc_out[(size_t)m * N + n] = (int32_t)v[r];
        if (y) y[(size_t)m * ldy + n] = f32_to_f16_bits((float)v[r] * sx[m] * swn);
      }
    }
  }
}

// Shared-ring variant for large grids: a 128 x 128 output tile per
// workgroup of NW waves, each computing a 64 x (128 / (NW / 2)) part of it over
// the workgroup's k blocks.  The waves copy every k block cooperatively (each
// issues 32 / NW of its whole-line LDS DMA reads, same swizzle as above) into
// a 4-stage ring shared by the workgroup, so three blocks (96 KB) are in
// flight while one is multiplied, and each block crosses L2 once per
// workgroup instead of once per wave.  One barrier per block: after it every
// wave's part of block j has landed and every wave is done with block j - 1,
// whose stage then receives block j + 3.
//
// Split along K (part != null): workgroup z of gridDim.z takes k blocks
// [z kbs, (z + 1) kbs) and stores its raw fp32 (int32) tile to part[z][m][n];
// gemm_splitk_reduce_kernel then sums the slices in order and scales.
template <bool FP8, int NW>
__global__ void __launch_bounds__(64 * NW) gemm_w8a8_ring_kernel(const uint8_t* __restrict__ xq,
                                                                 const float* __restrict__ sx, int M,
                                                                 const uint8_t* __restrict__ wq,
                                                                 const float* __restrict__ sw, int N, int K,
                                                                 uint16_t* __restrict__ y, int ldy,
                                                                 int32_t* __restrict__ acc_out, int kbs,
                                                                 void* __restrict__ part) {
  constexpr int BT = 128;                  // tile rows of x and of w
  constexpr int SA = BT * 128;             // bytes of one operand's k block
  constexpr int STAGE = 2 * SA;
  constexpr int NB = 4;
  constexpr int PER = 32 / NW;             // DMA instructions per wave per block
  constexpr int TB = 8 / NW * 2;           // 16-column blocks of a wave's part (4 or 2)
  typedef typename std::conditional<FP8, float4v, int4v>::type AccT;
  extern __shared__ uint4 lds4[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int m0 = blockIdx.y * BT;
  const int n0 = blockIdx.x * BT;
  const int kb0 = blockIdx.z * kbs;
  const int nkb = min(K >> 7, kb0 + kbs) - kb0;
  const int qm = wave / (NW / 2), qn = wave % (NW / 2);  // 64-row half, column part

  // this wave's DMA instructions: instruction g = wave * PER + u of the 32 a
  // block takes rows 8 (g % 16) .. + 7 of x (g < 16) or of w (g >= 16)
  const int drow = lane >> 3, dslot = lane & 7;
  const uint8_t* src[PER];
  uint32_t dst[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int g = wave * PER + u;
    const int r = 8 * (g & 15) + drow;
    const int seg = (dslot ^ (r & 7)) << 4;
    src[u] = g < 16 ? xq + (size_t)min(m0 + r, M - 1) * K + seg : wq + (size_t)min(n0 + r, N - 1) * K + seg;
    dst[u] = (g < 16 ? 0 : SA) + (g & 15) * 1024;
  }
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;
  auto dma = [&](int st, int kb) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint8_t* g = src[u] + (size_t)(kb0 + kb) * 128;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(ring + st * STAGE + dst[u]) : "memory", "m0");
    }
  };

  const int swz = r16 & 7;
  const int o0 = r16 * 128 + ((q ^ swz) << 4);
  const int o1 = r16 * 128 + (((q + 4) ^ swz) << 4);
  const uint8_t* abase = (const uint8_t*)lds4 + qm * 64 * 128;
  const uint8_t* bbase = (const uint8_t*)lds4 + SA + qn * (16 * TB) * 128;

  AccT acc[4][TB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = AccT{0, 0, 0, 0};

  auto compute = [&](int st) {
    uint4 fa[4][2], fb[TB][2];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      fa[a][0] = *(const uint4*)(abase + st * STAGE + a * 2048 + o0);
      fa[a][1] = *(const uint4*)(abase + st * STAGE + a * 2048 + o1);
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      fb[b][0] = *(const uint4*)(bbase + st * STAGE + b * 2048 + o0);
      fb[b][1] = *(const uint4*)(bbase + st * STAGE + b * 2048 + o1);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const uint4 al = fa[a][0], ah = fa[a][1];
        const uint4 bl = fb[b][0], bh = fb[b][1];
        if constexpr (FP8) {
          const int8v av = {(int)al.x, (int)al.y, (int)al.z, (int)al.w, (int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int8v bv = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w, (int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[a][b], 0, 0, 0, 0, 0, 0);
        } else {
          const int4v a0 = {(int)al.x, (int)al.y, (int)al.z, (int)al.w};
          const int4v b0 = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w};
          const int4v a1 = {(int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int4v b1 = {(int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[a][b], 0, 0, 0);
        }
      }
  };

#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (j < nkb) dma(j, j);
  for (int j = 0; j < nkb; ++j) {
    // this wave's DMAs of blocks after j that are already issued may stay in flight
    const int ahead = min(NB - 2, nkb - 1 - j);
    if (ahead >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * PER) : "memory");
    else if (ahead == 1)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's part of block j is in; block j - 1 is done
    if (j + NB - 1 < nkb) dma((j + NB - 1) % NB, j + NB - 1);
    compute(j % NB);
  }

  // epilogue: lane holds D[m = 4q + r][n = r16] of each 16 x 16 block
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int n = n0 + qn * (16 * TB) + b * 16 + r16;
    if (n >= N) continue;
    const float swn = (y && !part) ? sw[n] : 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + qm * 64 + a * 16 + 4 * q + r;
        if (m >= M) continue;
        if (part) {
          const size_t o = ((size_t)blockIdx.z * M + m) * N + n;
          if constexpr (FP8)
            ((float*)part)[o] = acc[a][b][r];
          else
            ((int32_t*)part)[o] = (int32_t)acc[a][b][r];
          continue;
        }
        if (acc_out) acc_out[(size_t)m * N + n] = (int32_t)acc[a][b][r];
        if (y) y[(size_t)m * ldy + n] = f32_to_f16_bits((float)acc[a][b][r] * sx[m] * swn);
      }
  }
}

// Large-tile variant for long prefill chunks: a 256 x 256 output tile per
// workgroup of eight waves, wave (qm, qn) computing rows 128 qm .. + 127 and
// columns 64 qn .. + 63 of it over all of K.  Every operand byte that reaches
// the compute unit feeds 256 outputs instead of 128, which halves the
// L2-to-LDS traffic per flop of the 128 x 128 ring; the price is LDS for only
// two stages of 64 KB (one k block multiplied while the next is copied).  The
// copy, swizzle and fragment reads are those of the ring kernel: 64 LDS DMA
// reads of 8 rows x 128 B per k block, eight per wave; one barrier per block
// tells that every wave's part of block j has landed and that block j - 1's
// stage is free for block j + 1.  Taken where the 256 x 256 tiles alone fill
// the 256 compute units (m >= 1024 with n >= 16384, for instance).
template <bool FP8>
__global__ void __launch_bounds__(512) gemm_w8a8_big_kernel(const uint8_t* __restrict__ xq,
                                                            const float* __restrict__ sx, int M,
                                                            const uint8_t* __restrict__ wq,
                                                            const float* __restrict__ sw, int N, int K,
                                                            uint16_t* __restrict__ y, int ldy,
                                                            int32_t* __restrict__ acc_out) {
  constexpr int BT = 256;                  // tile rows of x and of w
  constexpr int SA = BT * 128;             // bytes of one operand's k block
  constexpr int STAGE = 2 * SA;
  constexpr int PER = 8;                   // DMA instructions per wave per block (64 / 8 waves)
  typedef typename std::conditional<FP8, float4v, int4v>::type AccT;
  extern __shared__ uint4 lds4[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int m0 = blockIdx.y * BT;
  const int n0 = blockIdx.x * BT;
  const int nkb = K >> 7;
  const int qm = wave >> 2, qn = wave & 3;  // 128-row half, 64-column quarter

  // instruction g = wave * PER + u of a block takes rows 8 (g % 32) .. + 7
  // of x (g < 32) or of w (g >= 32)
  const int drow = lane >> 3, dslot = lane & 7;
  const uint8_t* src[PER];
  uint32_t dst[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int g = wave * PER + u;
    const int r = 8 * (g & 31) + drow;
    const int seg = (dslot ^ (r & 7)) << 4;
    src[u] = g < 32 ? xq + (size_t)min(m0 + r, M - 1) * K + seg : wq + (size_t)min(n0 + r, N - 1) * K + seg;
    dst[u] = (g < 32 ? 0 : SA) + (g & 31) * 1024;
  }
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;
  auto dma = [&](int st, int kb) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint8_t* g = src[u] + (size_t)kb * 128;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(ring + st * STAGE + dst[u]) : "memory", "m0");
    }
  };

  const int swz = r16 & 7;
  const int o0 = r16 * 128 + ((q ^ swz) << 4);
  const int o1 = r16 * 128 + (((q + 4) ^ swz) << 4);
  const uint8_t* abase = (const uint8_t*)lds4 + qm * 128 * 128;
  const uint8_t* bbase = (const uint8_t*)lds4 + SA + qn * 64 * 128;

  AccT acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = AccT{0, 0, 0, 0};

  auto compute = [&](int st) {
    uint4 fb[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      fb[b][0] = *(const uint4*)(bbase + st * STAGE + b * 2048 + o0);
      fb[b][1] = *(const uint4*)(bbase + st * STAGE + b * 2048 + o1);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const uint4 al = *(const uint4*)(abase + st * STAGE + a * 2048 + o0);
      const uint4 ah = *(const uint4*)(abase + st * STAGE + a * 2048 + o1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint4 bl = fb[b][0], bh = fb[b][1];
        if constexpr (FP8) {
          const int8v av = {(int)al.x, (int)al.y, (int)al.z, (int)al.w, (int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int8v bv = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w, (int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[a][b], 0, 0, 0, 0, 0, 0);
        } else {
          const int4v a0 = {(int)al.x, (int)al.y, (int)al.z, (int)al.w};
          const int4v b0 = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w};
          const int4v a1 = {(int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
          const int4v b1 = {(int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[a][b], 0, 0, 0);
        }
      }
    }
  };

  if (nkb > 0) dma(0, 0);
  for (int j = 0; j < nkb; ++j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of block j has landed
    __syncthreads();  // every wave's part of block j is in; block j - 1's stage is free
    if (j + 1 < nkb) dma((j + 1) & 1, j + 1);
    compute(j & 1);
  }

  // epilogue: lane holds D[m = 4q + r][n = r16] of each 16 x 16 block
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = n0 + qn * 64 + b * 16 + r16;
    if (n >= N) continue;
    const float swn = y ? sw[n] : 0.f;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + qm * 128 + a * 16 + 4 * q + r;
        if (m >= M) continue;
        if (acc_out) acc_out[(size_t)m * N + n] = (int32_t)acc[a][b][r];
        if (y) y[(size_t)m * ldy + n] = f32_to_f16_bits((float)acc[a][b][r] * sx[m] * swn);
      }
  }
}

// Split K, second step: the slices' tiles summed in slice order (fp32 for
// fp8, exact int32 for int8), then scaled, one thread per output.
template <bool FP8>
__global__ void __launch_bounds__(256) gemm_splitk_reduce_kernel(const void* __restrict__ part, int split,
                                                                 const float* __restrict__ sx, int M,
                                                                 const float* __restrict__ sw, int N,
                                                                 uint16_t* __restrict__ y, int ldy,
                                                                 int32_t* __restrict__ acc_out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t mn = (size_t)M * N;
  if (i >= mn) return;
  const int m = (int)(i / N), n = (int)(i - (size_t)m * N);
  // every slice's load is issued before the first add (split <= 16)
  uint32_t vals[16];
  const uint32_t* p = (const uint32_t*)part + i;
#pragma unroll
  for (int z = 0; z < 16; ++z) vals[z] = z < split ? p[(size_t)z * mn] : 0u;
  if constexpr (FP8) {
    float v = __builtin_bit_cast(float, vals[0]);
#pragma unroll
    for (int z = 1; z < 16; ++z)
      if (z < split) v += __builtin_bit_cast(float, vals[z]);
    y[(size_t)m * ldy + n] = f32_to_f16_bits(v * sx[m] * sw[n]);
  } else {
    int32_t v = (int32_t)vals[0];
#pragma unroll
    for (int z = 1; z < 16; ++z)
      if (z < split) v += (int32_t)vals[z];
    if (acc_out) acc_out[(size_t)m * N + n] = v;
    if (y) y[(size_t)m * ldy + n] = f32_to_f16_bits((float)v * sx[m] * sw[n]);
  }
}

// Tile shape: the largest of 64x64, 32x64, 32x32, 16x32 that still gives at
// least one workgroup per compute unit (256), else the smallest.
// blockIdx.x runs over n, so with N / BN a multiple of 8 the workgroups that
// share a weight tile land on the same XCD (dispatch is round-robin over 8).
template <bool FP8>
static void launch_ring(const void* xq, const float* sx, int m, const void* wq, const float* sw, int n, int k,
                        uint16_t* y, int ldy, int32_t* acc_out, int split, void* part, hipStream_t st) {
  constexpr int NW = 8;
  constexpr size_t lds = (size_t)4 * 2 * 128 * 128;
  static const bool attr_set = hipFuncSetAttribute((const void*)gemm_w8a8_ring_kernel<FP8, NW>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds) == hipSuccess;
  (void)attr_set;
  const int nkb = k >> 7;
  const int kbs = (nkb + split - 1) / split;
  const dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128), (unsigned)split);
  hipLaunchKernelGGL((gemm_w8a8_ring_kernel<FP8, NW>), grid, dim3(64 * NW), lds, st, (const uint8_t*)xq, sx, m,
                     (const uint8_t*)wq, sw, n, k, y, ldy, acc_out, kbs, part);
}

template <bool FP8>
static hipError_t launch_w8a8_t(const void* xq, const float* sx, int m, const void* wq, const float* sw,
                                int n, int k, uint16_t* y, int ldy, int32_t* acc_out, void* ws,
                                size_t ws_bytes, hipStream_t st) {
  // 128 x 128 tiles on a shared ring when they still make one workgroup per
  // compute unit
  // 256 x 256 tiles where they alone fill the compute units
  const long tiles256 = (long)((m + 255) / 256) * (long)((n + 255) / 256);
  if (tiles256 >= 256) {
    constexpr size_t lds = (size_t)2 * 2 * 256 * 128;
    static const bool attr_set = hipFuncSetAttribute((const void*)gemm_w8a8_big_kernel<FP8>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)lds) == hipSuccess;
    (void)attr_set;
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)((m + 255) / 256));
    hipLaunchKernelGGL((gemm_w8a8_big_kernel<FP8>), grid, dim3(512), lds, st, (const uint8_t*)xq, sx, m,
                       (const uint8_t*)wq, sw, n, k, y, ldy, acc_out);
    return hipGetLastError();
  }
  const long tiles128 = (long)((m + 127) / 128) * (long)((n + 127) / 128);
  if (tiles128 >= 256) {
    launch_ring<FP8>(xq, sx, m, wq, sw, n, k, y, ldy, acc_out, 1, nullptr, st);
    return hipGetLastError();
  }
  // fewer: split K over 2^s slices of at least 32 k blocks each until there
  // are 256 workgroups, when the tiles are full in m and the partial tiles
  // fit the workspace (shorter slices lose more to filling the ring and to
  // the partial tiles than the larger tiles save)
  {
    const int nkb = k >> 7;
    int split = 1;
    while (tiles128 * split < 256 && nkb / (2 * split) >= 32 && split < 16) split *= 2;
    if (m >= 128 && split > 1 && ws && (size_t)split * m * n * 4 <= ws_bytes) {
      launch_ring<FP8>(xq, sx, m, wq, sw, n, k, nullptr, 0, nullptr, split, ws, st);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      const size_t outs = (size_t)m * n;
      hipLaunchKernelGGL(gemm_splitk_reduce_kernel<FP8>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st,
                         (const void*)ws, split, sx, m, sw, n, y, ldy, acc_out);
      return hipGetLastError();
    }
  }
  struct Shape {
    int tm, tn;
  };
  const Shape shapes[] = {{4, 4}, {2, 4}, {2, 2}, {1, 2}};
  int pick = 3;
  for (int i = 0; i < 4; ++i) {
    const long wg = (long)((m + 16 * shapes[i].tm - 1) / (16 * shapes[i].tm)) *
                    (long)((n + 16 * shapes[i].tn - 1) / (16 * shapes[i].tn));
    if (wg >= 256) {
      pick = i;
      break;
    }
  }
  const int bm = 16 * shapes[pick].tm, bn = 16 * shapes[pick].tn;
  const dim3 grid((unsigned)((n + bn - 1) / bn), (unsigned)((m + bm - 1) / bm));
  const uint8_t* a = (const uint8_t*)xq;
  const uint8_t* b = (const uint8_t*)wq;
#define RQ_W8A8(TM, TN)                                                                              \
  {                                                                                                  \
    constexpr size_t lds = (size_t)4 * 2 * (16 * (TM) + 16 * (TN)) * 128;                            \
    static_assert(lds >= (size_t)4 * (TN) * 64 * 16, "reduction fits in the staging area");          \
    static const bool attr_set = hipFuncSetAttribute((const void*)gemm_w8a8_kernel<FP8, TM, TN, 4>,     \
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                                     (int)lds) == hipSuccess;                         \
    (void)attr_set;                                                                                  \
    hipLaunchKernelGGL((gemm_w8a8_kernel<FP8, TM, TN, 4>), grid, dim3(256), lds, st, a, sx, m, b, sw, n, \
                       k, y, ldy, acc_out);                                                          \
  }
  switch (pick) {
    case 0: RQ_W8A8(4, 4); break;
    case 1: RQ_W8A8(2, 4); break;
    case 2: RQ_W8A8(2, 2); break;
    default: RQ_W8A8(1, 2); break;
  }
#undef RQ_W8A8
  return hipGetLastError();
}

hipError_t launch_gemm_w8a8(const void* xq, const float* sx, int m, const void* wq, const float* sw,
                            int n, int k, bool fp8, uint16_t* y, int ldy, int32_t* acc_out, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (m == 0 || n == 0) return hipSuccess;
  if (fp8) return launch_w8a8_t<true>(xq, sx, m, wq, sw, n, k, y, ldy, acc_out, ws, ws_bytes, st);
  return launch_w8a8_t<false>(xq, sx, m, wq, sw, n, k, y, ldy, acc_out, ws, ws_bytes, st);
}

}  // namespace rq
