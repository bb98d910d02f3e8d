// Internal kernel launchers of librq (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

// ---- quantizers (quant.hip) ------------------------------------------------
// imp (may be null): fp32 [k] E[x^2] importances; non-null selects the
// activation-weighted scale search instead of RTN
// bits 5 / 6 also write the high plane `hi` (uint16 or uint8 per 8-k word)
hipError_t launch_quant_sym(const float* w, int64_t n, int64_t k, int bits, int group, void* codes,
                            uint16_t* scales, void* hi, int* flags, const float* imp, hipStream_t st);
hipError_t launch_quant_sb256(const float* w, int64_t n, int64_t k, void* qs, void* d, void* dmin,
                              void* sub, int* flags, const float* imp, hipStream_t st);
hipError_t launch_quant_rows_f32(const float* w, int64_t n, int64_t k, bool fp8, void* codes,
                                 float* scales, int* flags, hipStream_t st);
hipError_t launch_quant_rows_f16(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, bool fp8,
                                 void* codes, float* scales, int* flags, hipStream_t st);
hipError_t launch_to_f16(const float* w, int64_t count, uint16_t* out, int* flags, hipStream_t st);
hipError_t launch_to_bf16(const float* w, int64_t count, uint16_t* out, int* flags, hipStream_t st);

// ---- weight-streaming products, 1 <= m <= 32 (gemv.hip) ----------------------
enum GemvFormat { GF_W4 = 0, GF_W8 = 1, GF_SB = 2, GF_F16 = 3, GF_W5 = 4, GF_W6 = 5, GF_BF16 = 6 };

struct GemvMatrix {
  const void* codes;
  const uint16_t* scales;  // W4/W8: fp16 [n][k/g]; SB: d [n][k/256]
  const uint16_t* mins;    // SB: dmin [n][k/256]
  const uint32_t* sub;     // SB: [n][k/256][3] words; W6 / W5: high plane [n][k/8] (uint16 / uint8)
  const uint16_t* x;       // fp16 [m][ldx]
  uint16_t* y;             // fp16 [m][ldy]
  int n;
  int tiles;               // ceil(n / 16)
};

struct GemvBatch {
  GemvMatrix mat[3];
  int nmat;
  int k;
  int m;
  int ldx;
  int ldy;
  // caller's workspace for products split along K (null: no split): fp32
  // partial tiles (the planner keeps within ws_bytes), and one arrival
  // counter per tile group (zero between calls) through which, for a split
  // of up to four slices, the workgroup that finishes a tile group last finds
  // itself and adds the partial tiles (a second kernel adds more slices)
  float* ws;
  size_t ws_bytes;
  uint32_t* cnt;
};

// workspace size that admits every product's fastest plan
constexpr size_t kWorkspaceBytes = 64u << 20;
// The workspace starts with the arrival counters of the K-split weight-
// streaming products (one 32-bit word per tile group, zero whenever no call
// is running: zero-filled by the caller once, and every call leaves them at
// zero); the partial tiles of every product follow them.
constexpr size_t kSplitCounterBytes = 64u << 10;
constexpr int kSplitCounters = (int)(kSplitCounterBytes / 4);

hipError_t launch_gemv(const GemvBatch& b, int fmt, int group, hipStream_t st);

// The launch launch_gemv would make for b, computed on the host without
// touching the GPU (the same planners, in the same order).  false: no launch
// shape (launch_gemv returns hipErrorInvalidConfiguration).
struct GemvPlanInfo {
  int kernel;      // 1 streaming, 2 streaming with two k ranges, 3 streamed activations, 4 phased, 5 first version
  int split;       // K slices (> 1: partial tiles in the workspace, added in launch up to 4, else by a second kernel)
  int cps;         // chunks per slice (streaming, phased)
  int cpw;         // chunks per wave (streaming)
  int wpt;         // waves per row tile (streaming)
  int rt;          // row tiles per workgroup
  int workgroups;  // of the main launch
  int threads;     // per workgroup
  size_t lds;      // dynamic LDS of the main launch, bytes
  size_t ws_used;  // workspace bytes the partial tiles take (after the counters)
};
bool plan_gemv(const GemvBatch& b, int fmt, int group, GemvPlanInfo& out);

// ---- prefill products on int4 codes, any m (gemm_w4.hip) --------------------
struct W4Gemm {
  const uint16_t* x;       // fp16 [m][ldx]
  const uint8_t* codes;    // [n][k/2]
  const uint16_t* scales;  // symmetric: fp16 [n][k/group]; superblocks: d [n][k/256]
  const uint16_t* mins;    // superblocks: dmin [n][k/256]
  const uint8_t* sub;      // superblocks: [n][k/256][12]
  uint16_t* y;             // fp16 [m][ldy]
  int m, n, k, ldx, ldy;
};

// symmetric int4 (group 16, 32 or 64; k % 128 == 0) or, with sb, the
// asymmetric 256-superblocks (k % 256 == 0).  ws (may be null) is the
// stream's workspace of ws_bytes, for fp32 partial tiles when K is split.
hipError_t launch_gemm_w4(const W4Gemm& p, bool sb, int group, float* ws, size_t ws_bytes, hipStream_t st);

// ---- MFMA GEMMs on per-row quantized operands (gemm_mfma.hip) ---------------
// ws (may be null) is the stream's workspace of ws_bytes: shapes with fewer
// than 256 output tiles of 128 x 128 split K and keep partial tiles there.
hipError_t launch_gemm_w8a8(const void* xq, const float* sx, int m, const void* wq, const float* sw,
                            int n, int k, bool fp8, uint16_t* y, int ldy, int32_t* acc_out, void* ws,
                            size_t ws_bytes, hipStream_t st);

// ---- measurement aid (measure.hip) ------------------------------------------
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace rq
