// The librq C ABI (include/rq.h): validate, pick the kernel for the format
// and batch size, launch on the caller's stream.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include <vector>

#include "device_common.h"
#include "kernels.h"
#include "rq.h"
#include "validate.h"

using rqv::Span;

namespace {

inline hipStream_t S(void* s) { return (hipStream_t)s; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? RQ_OK : RQ_ERR_HIP; }

// launch_gemv: hipErrorInvalidConfiguration means no launch shape fits
// (activation slice too large for the LDS with no split-K workspace)
inline int gemv_status(hipError_t e) { return e == hipErrorInvalidConfiguration ? RQ_ERR_SHAPE : hip_status(e); }

// y must not overlap x or any weight buffer
int check_alias_out(const Span& y, const Span* ins, int nin) {
  for (int i = 0; i < nin; ++i)
    if (rqv::overlaps(y, ins[i])) return RQ_ERR_ALIAS;
  return RQ_OK;
}

int gemv_fmt(int format) {
  switch (format) {
    case RQ_W4_SYM: return rq::GF_W4;
    case RQ_W8_SYM: return rq::GF_W8;
    case RQ_W4_ASYM_SB256: return rq::GF_SB;
    case RQ_F16: return rq::GF_F16;
    case RQ_W5_SYM: return rq::GF_W5;
    case RQ_W6_SYM: return rq::GF_W6;
    case RQ_BF16: return rq::GF_BF16;
  }
  return -1;
}

void fill_matrix(rq::GemvMatrix& g, const rq_qweight* w, const uint16_t* x, uint16_t* y) {
  g.codes = w->codes;
  g.scales = (const uint16_t*)w->scales;
  g.mins = (const uint16_t*)w->mins;
  g.sub = (const uint32_t*)w->sub;
  g.x = x;
  g.y = y;
  g.n = (int)w->n;
  g.tiles = (int)((w->n + 15) / 16);
}

// The caller's workspace (may be NULL): 16-byte aligned, and disjoint from
// every input and output of the call.  RQ_OK or the error to return.
int check_ws(const void* ws, size_t ws_bytes, const Span* io, int nio) {
  if (!ws) return RQ_OK;
  if (!rqv::aligned16(ws)) return RQ_ERR_ALIGN;
  Span w;
  w.lo = (uintptr_t)ws;
  w.hi = w.lo + ws_bytes;
  for (int i = 0; i < nio; ++i)
    if (rqv::overlaps(w, io[i])) return RQ_ERR_ALIAS;
  return RQ_OK;
}

inline size_t ws_size(const void* ws, size_t ws_bytes) { return ws ? ws_bytes : 0; }

// The workspace's layout: rq::kSplitCounterBytes of arrival counters for
// the K-split weight-streaming products (zero whenever no call is running),
// then the partial tiles of every product.  A workspace that holds nothing
// past the counters counts as none.
inline bool ws_usable(const void* ws, size_t ws_bytes) { return ws && ws_bytes > rq::kSplitCounterBytes; }

void set_gemv_ws(rq::GemvBatch& b, void* ws, size_t ws_bytes) {
  if (ws_usable(ws, ws_bytes)) {
    b.cnt = (uint32_t*)ws;
    b.ws = (float*)((uint8_t*)ws + rq::kSplitCounterBytes);
    b.ws_bytes = ws_bytes - rq::kSplitCounterBytes;
  } else {
    b.cnt = nullptr;
    b.ws = nullptr;
    b.ws_bytes = 0;
  }
}

// partial tiles of the dense GEMMs: after the counters, which they leave alone
inline void* parts_of(void* ws, size_t ws_bytes) {
  return ws_usable(ws, ws_bytes) ? (void*)((uint8_t*)ws + rq::kSplitCounterBytes) : nullptr;
}
inline size_t parts_bytes(const void* ws, size_t ws_bytes) {
  return ws_usable(ws, ws_bytes) ? ws_bytes - rq::kSplitCounterBytes : 0;
}

// Scratch of rq_gemm_small_m_noalloc: the K-split partial sums live in this
// file-scope device array instead of a workspace, one copy per GPU, kept
// until the process ends.  Its host-side name is not a device address: the
// address of each GPU's copy is taken once, with that GPU current, by
// hipGetSymbolAddress, and only that address is handed to kernels.  It is
// laid out as a workspace: the split counters (zero-initialized with the
// array when the code object is loaded, and left at zero by every call),
// then 8 MiB for the partial tiles.
constexpr size_t kScratchParts = (size_t)8 << 20;
constexpr size_t kScratchBytes = rq::kSplitCounterBytes + kScratchParts;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's scratch address (nullptr on failure).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Shared path of the gemv entry points and rq_gemm_small_m.
// get_scratch (may be null): the workspace comes from it, once the arguments
// have passed validation
int small_m(const uint16_t* x, int64_t m, int64_t ldx, const rq_qweight* w, uint16_t* y, int64_t ldy,
            void* ws, size_t ws_bytes, void* stream, int want_format, int want_group,
            void* (*get_scratch)() = nullptr) {
  int st = rqv::check_weight(w);
  if (st != RQ_OK) return st;
  const int gf = gemv_fmt(w->format);
  if (gf < 0) return RQ_ERR_FORMAT;
  if (want_format && (w->format != want_format || (want_group && w->group != want_group)))
    return RQ_ERR_FORMAT;
  if (m < 0 || m > 32) return RQ_ERR_SHAPE;
  if ((st = rqv::check_act(x, m, w->k, ldx)) != RQ_OK) return st;
  if ((st = rqv::check_out(y, m, w->n, ldy)) != RQ_OK) return st;
  Span ins[6];
  rqv::weight_spans(w, ins);
  ins[4] = rqv::act_span(x, m, w->k, ldx, 2);
  ins[5] = rqv::act_span(y, m, w->n, ldy, 2);
  if ((st = check_alias_out(ins[5], ins, 5)) != RQ_OK) return st;
  if ((st = check_ws(ws, ws_bytes, ins, 6)) != RQ_OK) return st;
  if (m == 0 || w->n == 0) return RQ_OK;
  if (get_scratch) {
    ws = get_scratch();
    if (!ws) return RQ_ERR_HIP;
  }
  rq::GemvBatch b;
  memset(&b, 0, sizeof(b));
  fill_matrix(b.mat[0], w, x, y);
  b.nmat = 1;
  b.k = (int)w->k;
  b.m = (int)m;
  b.ldx = (int)ldx;
  b.ldy = (int)ldy;
  set_gemv_ws(b, ws, ws_size(ws, ws_bytes));
  return gemv_status(rq::launch_gemv(b, gf, w->group, S(stream)));
}

// rq_gemm_w4: int4 codes (symmetric groups or asymmetric superblocks), any m.
int gemm_w4(const uint16_t* x, int64_t m, int64_t ldx, const rq_qweight* w, uint16_t* y, int64_t ldy,
            void* ws, size_t ws_bytes, void* stream) {
  int st = rqv::check_weight(w);
  if (st != RQ_OK) return st;
  if (w->format != RQ_W4_SYM && w->format != RQ_W4_ASYM_SB256) return RQ_ERR_FORMAT;
  if (w->k % 128 != 0) return RQ_ERR_SHAPE;
  if (m < 0 || m >= rqv::kMaxDim) return RQ_ERR_SHAPE;
  if ((st = rqv::check_act(x, m, w->k, ldx)) != RQ_OK) return st;
  if ((st = rqv::check_out(y, m, w->n, ldy)) != RQ_OK) return st;
  Span ins[6];
  rqv::weight_spans(w, ins);
  ins[4] = rqv::act_span(x, m, w->k, ldx, 2);
  ins[5] = rqv::act_span(y, m, w->n, ldy, 2);
  if ((st = check_alias_out(ins[5], ins, 5)) != RQ_OK) return st;
  if ((st = check_ws(ws, ws_bytes, ins, 6)) != RQ_OK) return st;
  if (m == 0 || w->n == 0) return RQ_OK;
  rq::W4Gemm p;
  p.x = x;
  p.codes = (const uint8_t*)w->codes;
  p.scales = (const uint16_t*)w->scales;
  p.mins = (const uint16_t*)w->mins;
  p.sub = (const uint8_t*)w->sub;
  p.y = y;
  p.m = (int)m;
  p.n = (int)w->n;
  p.k = (int)w->k;
  p.ldx = (int)ldx;
  p.ldy = (int)ldy;
  return hip_status(rq::launch_gemm_w4(p, w->format == RQ_W4_ASYM_SB256, w->group, (float*)parts_of(ws, ws_bytes),
                                       parts_bytes(ws, ws_bytes), S(stream)));
}

int w8a8(const void* xq, const float* sx, int64_t m, const rq_qweight* w, uint16_t* y, int64_t ldy,
         int32_t* acc, void* ws, size_t ws_bytes, void* stream, int want_format) {
  int st = rqv::check_weight(w);
  if (st != RQ_OK) return st;
  if (w->format != want_format) return RQ_ERR_FORMAT;
  if (w->k % 128 != 0) return RQ_ERR_SHAPE;
  if (want_format == RQ_I8_CH && w->k > 131072) return RQ_ERR_SHAPE;
  if (!xq || (y && !sx)) return RQ_ERR_NULL;
  if (m < 0 || m >= rqv::kMaxDim) return RQ_ERR_SHAPE;
  if (!rqv::aligned16(xq) || (sx && !rqv::aligned16(sx))) return RQ_ERR_ALIGN;
  Span ins[8];
  rqv::weight_spans(w, ins);
  ins[4] = rqv::act_span(xq, m, w->k, w->k, 1);
  ins[5] = sx ? rqv::act_span(sx, m > 0 ? 1 : 0, m, m, 4) : Span();
  if (y) {
    if ((st = rqv::check_out(y, m, w->n, ldy)) != RQ_OK) return st;
    ins[6] = rqv::act_span(y, m, w->n, ldy, 2);
    if ((st = check_alias_out(ins[6], ins, 6)) != RQ_OK) return st;
  }
  if (acc) {
    if (!rqv::aligned16(acc)) return RQ_ERR_ALIGN;
    ins[7] = rqv::act_span(acc, m, w->n, w->n, 4);
    if ((st = check_alias_out(ins[7], ins, 6)) != RQ_OK) return st;
  }
  if ((st = check_ws(ws, ws_bytes, ins, 8)) != RQ_OK) return st;
  if (m == 0 || w->n == 0) return RQ_OK;
  return hip_status(rq::launch_gemm_w8a8(xq, sx, (int)m, w->codes, (const float*)w->scales, (int)w->n,
                                         (int)w->k, want_format == RQ_FP8_E4M3_CH, y, (int)ldy, acc,
                                         parts_of(ws, ws_bytes), parts_bytes(ws, ws_bytes), S(stream)));
}

}  // namespace

extern "C" {

int rq_abi_version(void) { return RQ_ABI_VERSION; }

const char* rq_status_str(int status) {
  switch (status) {
    case RQ_OK: return "ok";
    case RQ_ERR_NULL: return "null pointer";
    case RQ_ERR_SHAPE: return "bad shape or leading dimension";
    case RQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case RQ_ERR_FORMAT: return "unknown format/group or wrong entry point for the format";
    case RQ_ERR_NONFINITE: return "non-finite input";
    case RQ_ERR_RANGE: return "scale overflows its storage type";
    case RQ_ERR_HIP: return "HIP runtime error";
    case RQ_ERR_ALIAS: return "output overlaps an input";
    case RQ_ERR_SCRATCH: return "needs more than the static scratch of rq_gemm_small_m_noalloc";
    case RQ_ERR_DEGENERATE: return "every weight is equal: no gap to normalise";
  }
  return "unknown status";
}

int rq_qweight_bytes(int format, int group, int64_t n, int64_t k, size_t* codes, size_t* scales,
                     size_t* mins, size_t* sub) {
  return rqv::weight_bytes(format, group, n, k, codes, scales, mins, sub);
}

namespace {
// Shared path of rq_quantize_rtn and rq_quantize_aw (imp non-null).
int quantize_impl(const float* w, const float* imp, const rq_qweight* out, void* stream) {
  if (!w) return RQ_ERR_NULL;
  int st = rqv::check_weight(out);
  if (st != RQ_OK) return st;
  if (!rqv::aligned16(w) || (imp && !rqv::aligned16(imp))) return RQ_ERR_ALIGN;
  Span outs[4];
  rqv::weight_spans(out, outs);
  const Span in = rqv::act_span(w, out->n, out->k, out->k, 4);
  const Span ins = imp ? rqv::act_span(imp, 1, out->k, out->k, 4) : Span();
  for (int i = 0; i < 4; ++i)
    if (rqv::overlaps(in, outs[i]) || rqv::overlaps(ins, outs[i])) return RQ_ERR_ALIAS;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (rqv::overlaps(outs[i], outs[j])) return RQ_ERR_ALIAS;
  if (out->n == 0) return RQ_OK;
  hipStream_t s = S(stream);
  int* flags = nullptr;
  if (hipMallocAsync((void**)&flags, 2 * sizeof(int), s) != hipSuccess) return RQ_ERR_HIP;
  hipError_t e = hipMemsetAsync(flags, 0, 2 * sizeof(int), s);
  const int64_t n = out->n, k = out->k;
  if (e == hipSuccess) {
    switch (out->format) {
      case RQ_W8_SYM:
      case RQ_W4_SYM:
        e = rq::launch_quant_sym(w, n, k, out->format == RQ_W8_SYM ? 8 : 4, out->group, out->codes,
                                 (uint16_t*)out->scales, nullptr, flags, imp, s);
        break;
      case RQ_W6_SYM:
      case RQ_W5_SYM:
        e = rq::launch_quant_sym(w, n, k, out->format == RQ_W6_SYM ? 6 : 5, out->group, out->codes,
                                 (uint16_t*)out->scales, out->sub, flags, imp, s);
        break;
      case RQ_BF16:
        e = rq::launch_to_bf16(w, n * k, (uint16_t*)out->codes, flags, s);
        break;
      case RQ_W4_ASYM_SB256:
        e = rq::launch_quant_sb256(w, n, k, out->codes, out->scales, out->mins, out->sub, flags, imp, s);
        break;
      case RQ_FP8_E4M3_CH:
      case RQ_I8_CH:
        e = rq::launch_quant_rows_f32(w, n, k, out->format == RQ_FP8_E4M3_CH, out->codes,
                                      (float*)out->scales, flags, s);
        break;
      case RQ_F16:
        e = rq::launch_to_f16(w, n * k, (uint16_t*)out->codes, flags, s);
        break;
    }
  }
  int host[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(host, flags, sizeof(host), hipMemcpyDeviceToHost, s);
  hipError_t ef = hipFreeAsync(flags, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return RQ_ERR_HIP;
  if (host[0]) return RQ_ERR_NONFINITE;
  if (host[1]) return RQ_ERR_RANGE;
  return RQ_OK;
}
}  // namespace

int rq_quantize_rtn(const float* w, const rq_qweight* out, void* stream) {
  return quantize_impl(w, nullptr, out, stream);
}

int rq_quantize_aw(const float* w, const float* act_sq, const rq_qweight* out, void* stream) {
  if (!act_sq || !out) return RQ_ERR_NULL;
  if (out->format != RQ_W8_SYM && out->format != RQ_W4_SYM && out->format != RQ_W4_ASYM_SB256 &&
      out->format != RQ_W6_SYM && out->format != RQ_W5_SYM)
    return RQ_ERR_FORMAT;
  return quantize_impl(w, act_sq, out, stream);
}

#define RQ_GEMV_ENTRY(NAME, FORMAT, GROUP)                                                           \
  int NAME(const uint16_t* x, const rq_qweight* w, uint16_t* y, void* ws, size_t ws_bytes, void* stream) { \
    if (!w) return RQ_ERR_NULL;                                                                      \
    return small_m(x, 1, w->k + (8 - w->k % 8) % 8, w, y, w->n > 0 ? w->n : 1, ws, ws_bytes, stream,   \
                   FORMAT, GROUP);                                                                   \
  }

RQ_GEMV_ENTRY(rq_gemv_w4g16, RQ_W4_SYM, 16)
RQ_GEMV_ENTRY(rq_gemv_w4g32, RQ_W4_SYM, 32)
RQ_GEMV_ENTRY(rq_gemv_w4g64, RQ_W4_SYM, 64)
RQ_GEMV_ENTRY(rq_gemv_w8g16, RQ_W8_SYM, 16)
RQ_GEMV_ENTRY(rq_gemv_w8g32, RQ_W8_SYM, 32)
RQ_GEMV_ENTRY(rq_gemv_w8g64, RQ_W8_SYM, 64)
RQ_GEMV_ENTRY(rq_gemv_w4sb256, RQ_W4_ASYM_SB256, 32)
RQ_GEMV_ENTRY(rq_gemv_f16, RQ_F16, 0)
#undef RQ_GEMV_ENTRY

int rq_gemm_small_m(const uint16_t* x, int64_t m, int64_t ldx, const rq_qweight* w, uint16_t* y,
                    int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return small_m(x, m, ldx, w, y, ldy, ws, ws_bytes, stream, 0, 0);
}

int rq_plan_small_m(const rq_qweight* w, int64_t m, int64_t ldx, size_t ws_bytes, rq_plan* out) {
  if (!out) return RQ_ERR_NULL;
  memset(out, 0, sizeof(*out));
  int st = rqv::check_weight(w);
  if (st != RQ_OK) return st;
  const int gf = gemv_fmt(w->format);
  if (gf < 0) return RQ_ERR_FORMAT;
  if (m < 0 || m > 32) return RQ_ERR_SHAPE;
  // x's shape and stride checks, as rq_gemm_small_m makes them (the address
  // stands for any aligned activation buffer)
  if ((st = rqv::check_act((const void*)(uintptr_t)256, m, w->k, ldx)) != RQ_OK) return st;
  if (m == 0 || w->n == 0) return RQ_OK;
  rq::GemvBatch b;
  memset(&b, 0, sizeof(b));
  b.mat[0].n = (int)w->n;
  b.mat[0].tiles = (int)((w->n + 15) / 16);
  b.nmat = 1;
  b.k = (int)w->k;
  b.m = (int)m;
  b.ldx = (int)ldx;
  b.ldy = (int)w->n;
  // the planner only asks whether a workspace exists and how large it is
  set_gemv_ws(b, ws_bytes ? (void*)(uintptr_t)256 : nullptr, ws_bytes);
  rq::GemvPlanInfo p;
  if (!rq::plan_gemv(b, gf, w->group, p)) return RQ_ERR_SHAPE;
  out->kernel = p.kernel;
  out->split = p.split;
  out->chunks_per_slice = p.cps;
  out->chunks_per_wave = p.cpw;
  out->waves_per_tile = p.wpt;
  out->tiles_per_workgroup = p.rt;
  out->workgroups = p.workgroups;
  out->threads = p.threads;
  out->lds_bytes = (int64_t)p.lds;
  out->workspace_bytes = (int64_t)(p.split > 1 ? rq::kSplitCounterBytes + p.ws_used : 0);
  return RQ_OK;
}

int rq_fused_rkv(const uint16_t* xr, const uint16_t* xk, const uint16_t* xv, int64_t m, int64_t ldx,
                 const rq_qweight* wr, const rq_qweight* wk, const rq_qweight* wv, uint16_t* yr,
                 uint16_t* yk, uint16_t* yv, int64_t ldy, void* wsp, size_t ws_bytes, void* stream) {
  const rq_qweight* ws[3] = {wr, wk, wv};
  const uint16_t* xs[3] = {xr, xk, xv};
  uint16_t* ys[3] = {yr, yk, yv};
  int st;
  for (int i = 0; i < 3; ++i)
    if ((st = rqv::check_weight(ws[i])) != RQ_OK) return st;
  const int gf = gemv_fmt(wr->format);
  if (gf < 0) return RQ_ERR_FORMAT;
  for (int i = 1; i < 3; ++i)
    if (ws[i]->format != wr->format || ws[i]->group != wr->group) return RQ_ERR_FORMAT;
  for (int i = 1; i < 3; ++i)
    if (ws[i]->k != wr->k) return RQ_ERR_SHAPE;
  if (m < 0 || m > 32) return RQ_ERR_SHAPE;
  Span ins[15];
  for (int i = 0; i < 3; ++i) {
    if ((st = rqv::check_act(xs[i], m, wr->k, ldx)) != RQ_OK) return st;
    if ((st = rqv::check_out(ys[i], m, ws[i]->n, ldy)) != RQ_OK) return st;
    rqv::weight_spans(ws[i], ins + 4 * i);
    ins[12 + i] = rqv::act_span(xs[i], m, wr->k, ldx, 2);
  }
  Span outs[3];
  for (int i = 0; i < 3; ++i) outs[i] = rqv::act_span(ys[i], m, ws[i]->n, ldy, 2);
  for (int i = 0; i < 3; ++i) {
    if ((st = check_alias_out(outs[i], ins, 15)) != RQ_OK) return st;
    for (int j = i + 1; j < 3; ++j)
      if (rqv::overlaps(outs[i], outs[j])) return RQ_ERR_ALIAS;
  }
  if ((st = check_ws(wsp, ws_bytes, ins, 15)) != RQ_OK) return st;
  if ((st = check_ws(wsp, ws_bytes, outs, 3)) != RQ_OK) return st;
  if (m == 0) return RQ_OK;
  rq::GemvBatch b;
  memset(&b, 0, sizeof(b));
  b.nmat = 3;
  for (int i = 0; i < 3; ++i) fill_matrix(b.mat[i], ws[i], xs[i], ys[i]);
  b.k = (int)wr->k;
  b.m = (int)m;
  b.ldx = (int)ldx;
  b.ldy = (int)ldy;
  set_gemv_ws(b, wsp, ws_size(wsp, ws_bytes));
  return gemv_status(rq::launch_gemv(b, gf, wr->group, S(stream)));
}

int rq_quantize_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, int format, void* xq,
                    float* sx, void* stream) {
  if (format != RQ_FP8_E4M3_CH && format != RQ_I8_CH) return RQ_ERR_FORMAT;
  int st = rqv::check_act(x, m, k, ldx);
  if (st != RQ_OK) return st;
  if (!xq || !sx) return RQ_ERR_NULL;
  if (k % 16 != 0) return RQ_ERR_SHAPE;
  if (!rqv::aligned16(xq) || !rqv::aligned16(sx)) return RQ_ERR_ALIGN;
  const Span in = rqv::act_span(x, m, k, ldx, 2);
  const Span o1 = rqv::act_span(xq, m, k, k, 1);
  const Span o2 = rqv::act_span(sx, m > 0 ? 1 : 0, m, m, 4);
  if (rqv::overlaps(in, o1) || rqv::overlaps(in, o2) || rqv::overlaps(o1, o2)) return RQ_ERR_ALIAS;
  if (m == 0) return RQ_OK;
  return hip_status(
      rq::launch_quant_rows_f16(x, m, k, ldx, format == RQ_FP8_E4M3_CH, xq, sx, nullptr, S(stream)));
}

int rq_gemm_w4(const uint16_t* x, int64_t m, int64_t ldx, const rq_qweight* w, uint16_t* y, int64_t ldy,
               void* ws, size_t ws_bytes, void* stream) {
  return gemm_w4(x, m, ldx, w, y, ldy, ws, ws_bytes, stream);
}

int rq_gemm_fp8(const uint8_t* xq, const float* sx, int64_t m, const rq_qweight* w, uint16_t* y,
                int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  if (!y) return RQ_ERR_NULL;
  return w8a8(xq, sx, m, w, y, ldy, nullptr, ws, ws_bytes, stream, RQ_FP8_E4M3_CH);
}

int rq_gemm_int8(const int8_t* xq, const float* sx, int64_t m, const rq_qweight* w, uint16_t* y,
                 int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  if (!y) return RQ_ERR_NULL;
  return w8a8(xq, sx, m, w, y, ldy, nullptr, ws, ws_bytes, stream, RQ_I8_CH);
}

int rq_gemm_int8_acc(const int8_t* xq, int64_t m, const rq_qweight* w, int32_t* acc, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!acc || !w) return RQ_ERR_NULL;
  return w8a8(xq, nullptr, m, w, nullptr, w->n, acc, ws, ws_bytes, stream, RQ_I8_CH);
}

size_t rq_workspace_bytes(void) { return rq::kWorkspaceBytes; }

int rq_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return RQ_ERR_NULL;
  if (!rqv::aligned16(buf) || ((uintptr_t)sink & 3u)) return RQ_ERR_ALIGN;
  if (bytes % 16 != 0) return RQ_ERR_SHAPE;
  return hip_status(rq::launch_stream_read(buf, bytes, sink, S(stream)));
}

int rq_gemm_small_m_noalloc(const uint16_t* x, int64_t m, int64_t ldx, const rq_qweight* w, uint16_t* y,
                            int64_t ldy, void* stream) {
  if (!w) return RQ_ERR_NULL;
  // every launch shape of this product keeps its partial sums within the
  // scratch: at most 16 K slices of 16-row tiles, each tile 1 KiB per
  // 16 activation rows (so the plan equals that of a full workspace)
  const int64_t mt = m <= 16 ? 1 : 2;
  if (w->n > 0 && 16 * ((w->n + 15) / 16) * mt * 1024 > (int64_t)kScratchParts) return RQ_ERR_SCRATCH;
  return small_m(x, m, ldx, w, y, ldy, nullptr, kScratchBytes, stream, 0, 0, scratch_address);
}

int rq_host_convert(int kind, const double* in, void* out, int64_t count) {
  if (!in || !out) return RQ_ERR_NULL;
  if (count < 0) return RQ_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) {
    switch (kind) {
      case 0: ((uint16_t*)out)[i] = rq::f64_to_f16_bits(in[i]); break;
      case 1: ((uint32_t*)out)[i] = rq::f64_to_f32_bits(in[i]); break;
      case 2: ((uint8_t*)out)[i] = rq::f64_to_e4m3(in[i]); break;
      default: return RQ_ERR_FORMAT;
    }
  }
  return RQ_OK;
}

}  // extern "C"
