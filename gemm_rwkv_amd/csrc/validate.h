// Argument validation of the librq C ABI: pure host C++, no HIP calls, so it
// can be exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rq.h"

namespace rqv {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // n, k, m, ld below this

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

bool overlaps(const Span& a, const Span& b);

// RQ_OK or RQ_ERR_FORMAT for an unknown format or a group it does not allow.
int check_format(int format, int group);

// Shape rules of a (format, group, n, k) weight; RQ_OK / RQ_ERR_FORMAT / RQ_ERR_SHAPE.
int check_shape(int format, int group, int64_t n, int64_t k);

int weight_bytes(int format, int group, int64_t n, int64_t k, size_t* codes, size_t* scales,
                 size_t* mins, size_t* sub);

// Full descriptor check: NULLs, format, shape, alignment.
int check_weight(const rq_qweight* w);

// The device memory a weight occupies (codes, scales, mins, sub).
void weight_spans(const rq_qweight* w, Span out[4]);

// fp16 activations x[m][ldx] (k used per row): NULL, shape, alignment.
int check_act(const void* x, int64_t m, int64_t k, int64_t ldx);
Span act_span(const void* x, int64_t m, int64_t k, int64_t ldx, int64_t elem);

// fp16 outputs y[m][ldy] (n used per row).
int check_out(const void* y, int64_t m, int64_t n, int64_t ldy);

bool aligned16(const void* p);

}  // namespace rqv
