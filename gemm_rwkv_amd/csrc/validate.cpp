// Argument validation of the librq C ABI (host C++ only).
#include "validate.h"

namespace rqv {

bool overlaps(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_format(int format, int group) {
  switch (format) {
    case RQ_W8_SYM:
    case RQ_W4_SYM:
      return (group == 16 || group == 32 || group == 64) ? RQ_OK : RQ_ERR_FORMAT;
    case RQ_W6_SYM:
    case RQ_W5_SYM:
      return (group == 32 || group == 64) ? RQ_OK : RQ_ERR_FORMAT;
    case RQ_W4_ASYM_SB256:
      return group == 32 ? RQ_OK : RQ_ERR_FORMAT;
    case RQ_FP8_E4M3_CH:
    case RQ_I8_CH:
    case RQ_F16:
    case RQ_BF16:
      return RQ_OK;
    default:
      return RQ_ERR_FORMAT;
  }
}

int check_shape(int format, int group, int64_t n, int64_t k) {
  int st = check_format(format, group);
  if (st != RQ_OK) return st;
  if (n < 0 || n >= kMaxDim || k < 1 || k >= kMaxDim) return RQ_ERR_SHAPE;
  switch (format) {
    case RQ_W8_SYM:
    case RQ_W4_SYM:
      return (k % group == 0) ? RQ_OK : RQ_ERR_SHAPE;
    case RQ_W6_SYM:
    case RQ_W5_SYM:
      return (k % 128 == 0) ? RQ_OK : RQ_ERR_SHAPE;
    case RQ_W4_ASYM_SB256:
      return (k % 256 == 0) ? RQ_OK : RQ_ERR_SHAPE;
    case RQ_FP8_E4M3_CH:
    case RQ_I8_CH:
      return (k % 16 == 0) ? RQ_OK : RQ_ERR_SHAPE;
    case RQ_F16:
      return (k % 8 == 0) ? RQ_OK : RQ_ERR_SHAPE;
    case RQ_BF16:
      return (k % 32 == 0) ? RQ_OK : RQ_ERR_SHAPE;
  }
  return RQ_ERR_FORMAT;
}

int weight_bytes(int format, int group, int64_t n, int64_t k, size_t* codes, size_t* scales,
                 size_t* mins, size_t* sub) {
  int st = check_shape(format, group, n, k);
  if (st != RQ_OK) return st;
  const size_t N = (size_t)n, K = (size_t)k;
  size_t c = 0, s = 0, m = 0, b = 0;
  switch (format) {
    case RQ_W8_SYM:
      c = N * K;
      s = N * (K / (size_t)group) * 2;
      break;
    case RQ_W4_SYM:
      c = N * K / 2;
      s = N * (K / (size_t)group) * 2;
      break;
    case RQ_W4_ASYM_SB256:
      c = N * K / 2;
      s = N * (K / 256) * 2;
      m = s;
      b = N * (K / 256) * 12;
      break;
    case RQ_FP8_E4M3_CH:
    case RQ_I8_CH:
      c = N * K;
      s = N * 4;
      break;
    case RQ_W6_SYM:
    case RQ_W5_SYM:
      c = N * K / 2;
      s = N * (K / (size_t)group) * 2;
      b = N * (K / 8) * (format == RQ_W6_SYM ? 2 : 1);
      break;
    case RQ_F16:
    case RQ_BF16:
      c = N * K * 2;
      break;
  }
  if (codes) *codes = c;
  if (scales) *scales = s;
  if (mins) *mins = m;
  if (sub) *sub = b;
  return RQ_OK;
}

int check_weight(const rq_qweight* w) {
  if (!w) return RQ_ERR_NULL;
  int st = check_format(w->format, w->group);
  if (st != RQ_OK) return st;
  if (!w->codes) return RQ_ERR_NULL;
  const bool plain = w->format == RQ_F16 || w->format == RQ_BF16;
  const bool two_plane = w->format == RQ_W6_SYM || w->format == RQ_W5_SYM;
  if (!plain && !w->scales) return RQ_ERR_NULL;
  if (w->format == RQ_W4_ASYM_SB256 && (!w->mins || !w->sub)) return RQ_ERR_NULL;
  if (two_plane && !w->sub) return RQ_ERR_NULL;
  st = check_shape(w->format, w->group, w->n, w->k);
  if (st != RQ_OK) return st;
  if (!aligned16(w->codes)) return RQ_ERR_ALIGN;
  if (!plain && !aligned16(w->scales)) return RQ_ERR_ALIGN;
  if (w->format == RQ_W4_ASYM_SB256 && (!aligned16(w->mins) || !aligned16(w->sub)))
    return RQ_ERR_ALIGN;
  if (two_plane && !aligned16(w->sub)) return RQ_ERR_ALIGN;
  return RQ_OK;
}

void weight_spans(const rq_qweight* w, Span out[4]) {
  size_t b[4] = {0, 0, 0, 0};
  weight_bytes(w->format, w->group, w->n, w->k, &b[0], &b[1], &b[2], &b[3]);
  void* p[4] = {w->codes, w->scales, w->mins, w->sub};
  for (int i = 0; i < 4; ++i) {
    out[i].lo = (uintptr_t)p[i];
    out[i].hi = p[i] ? (uintptr_t)p[i] + b[i] : (uintptr_t)p[i];
  }
}

int check_act(const void* x, int64_t m, int64_t k, int64_t ldx) {
  if (!x) return RQ_ERR_NULL;
  if (m < 0 || m >= kMaxDim || k < 1 || k >= kMaxDim || ldx < k || ldx >= kMaxDim)
    return RQ_ERR_SHAPE;
  if (m * ldx >= ((int64_t)1 << 40)) return RQ_ERR_SHAPE;
  if (!aligned16(x) || (ldx % 8) != 0) return RQ_ERR_ALIGN;
  return RQ_OK;
}

Span act_span(const void* x, int64_t m, int64_t k, int64_t ldx, int64_t elem) {
  Span s;
  s.lo = (uintptr_t)x;
  s.hi = m > 0 ? (uintptr_t)x + (size_t)((m - 1) * ldx + k) * (size_t)elem : s.lo;
  return s;
}

int check_out(const void* y, int64_t m, int64_t n, int64_t ldy) {
  if (!y) return RQ_ERR_NULL;
  if (m < 0 || m >= kMaxDim || n < 0 || n >= kMaxDim || ldy < n || ldy < 1 || ldy >= kMaxDim)
    return RQ_ERR_SHAPE;
  if (m * ldy >= ((int64_t)1 << 40)) return RQ_ERR_SHAPE;
  if (!aligned16(y)) return RQ_ERR_ALIGN;
  return RQ_OK;
}

}  // namespace rqv
