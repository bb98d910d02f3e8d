// Decode chain: a sequence of dependent weight-streaming products, M = 1, run
// by one persistent launch.
//
// A decode step of an RWKV-7 model is a chain of matrix-vector products where
// each product's input is an earlier product's output (the fused R/K/V, then
// the output projection, then the channel-mix key and value, layer after
// layer, then the head: model card "RWKV-7 G1 1.5B -- int4 GPTQ for
// rwkv-sglang", summary: int4 GEMV family, decode at batch <= 32).  One
// launch per product leaves the weight stream idle at every launch boundary
// (dispatch, ramp-up, tail).  Here one workgroup per compute unit walks the
// whole chain and keeps loading weights across the boundaries: a product's
// weights do not depend on its input, only the multiply does.
//
// Work split.  Product q runs on an R x S grid of workgroups (w = r * S + s):
// row block r (rows/16 tiles of 16 rows) times K slice s.  A workgroup's
// result over its slice is an fp16 partial sum, part[s][row]; a consumer
// workgroup whose own K slice covers rows [lo, lo + L) of that output waits
// only for the producers of those rows (the S workgroups of the covering row
// blocks, about 16 rather than all 256) and adds their partials in slice order
// (fp32) into its fp16 input slice.  The first consumer's row-block-0
// workgroups also store that slice as the product's fp16 output; outputs that
// no later product reads are finalized the same way by a last pass (FIN).
// With S = 1 a workgroup covers all of K and stores the fp16 output itself.
//
// Waves.  Eight compute waves and one communication wave per workgroup.
//   * A compute wave owns tiles (or K parts of a tile) of each product and
//     streams their code chunks (16 rows x 64 bytes) and scales by LDS DMA
//     into its own ring of 12 slots, non-temporal, running ahead across
//     product boundaries; it waits for a slot with a fixed vmcnt (two DMA
//     instructions per chunk, dummies past the end), decodes the codes to
//     exact fp16 integers and multiplies on v_mfma_f32_16x16x32_f16 with the
//     input as the A operand (row 0; rows 1..15 zero), scaling each 64-group
//     in fp32.  Its results go to LDS.  It never waits for its own loads
//     except through the ring, so it does no global stores.
//   * The communication wave stores each product's results (agent-scope
//     stores), waits for them, and publishes flag[q][w] = epoch; it then
//     polls the producers of the next input (agent-scope loads, bounded),
//     and copies their partials into LDS by DMA.  All waves add them.
// Three barriers per product (input copied, input ready, results ready)
// order the LDS use; every wave passes every barrier.
//
// Memory model.  Results, partials and flags are written with agent-scope
// (sc1) stores and read with agent-scope loads, which the hardware keeps
// coherent across the XCDs' L2 caches; a producer waits for its stores to
// complete (vmcnt 0) before it stores its flag, and a consumer reads data
// only after it has seen every flag it needs.  The epoch (read from device
// memory at the start of a launch and advanced by a second, one-thread
// kernel after it) tells this launch's flags from older ones, so a captured
// graph can replay the pair.
//
// Termination.  Every wait is bounded (kSpinMax polls); on expiry the wave
// records an error word, stops waiting for the rest of the launch (its
// results are then unspecified) and still passes every barrier, so the
// launch always ends.  All workgroups are resident at once (one per compute
// unit, LDS-limited), so no wait depends on a workgroup that cannot run.
#include <hip/hip_runtime.h>
#include <string.h>

#include <utility>
#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace rq {

namespace {

constexpr int kWG = kChainWorkgroups;  // 256
constexpr int kCW = 8;                 // compute waves
constexpr int kThreads = (kCW + 1) * 64;
constexpr int kSlots = 12;
constexpr int kSlotCode = 1024, kSlotScale = 128, kSlot = kSlotCode + kSlotScale;
constexpr int kRingBytes = kCW * kSlots * kSlot;  // 110592
constexpr int kStageBytes = 32768;                // input slice and partial staging
constexpr int kPartBytes = 4096;                  // per-tile results, fp32
constexpr int kLdsBytes = kRingBytes + kStageBytes + kPartBytes;
constexpr int kSpinMax = 1 << 21;
constexpr uint32_t kOOB = 0x80000000u;            // buffer offset past any range: reads zero

enum { kFmtW4 = 0, kFmtF16 = 1, kFmtFin = 2 };

struct Op {
  const uint8_t* codes;    // int4 g64 code words [n][k/2], or fp16 [n][k]
  const uint16_t* scales;  // fp16 [n][k/64]
  uint16_t* y;             // fp16 output [n]
  uint16_t* part;          // fp16 partials [S][n] (S > 1)
  const uint16_t* xext;    // input [k] when src < 0
  int fmt, n, k;
  int R, S, rows, kslice;
  int src;                 // producer of the input, -1: xext
  int src_S, src_rows, src_n;
  uint16_t* src_y;
  const uint16_t* src_part;
  int fin_src;             // row-block-0 workgroups store the reduced input as src's output
  int x_keep;              // same input slice as the previous product: keep it in LDS
  int tiles_w, chunks_w, wpt;
  int fin_lo, fin_hi;      // FIN: its targets
};

struct Target {
  uint16_t* y;
  const uint16_t* part;
  int op, n, S, rows;
};

struct Plan {
  int nops = 0;         // including FIN
  int m = 1;
  Op* d_ops = nullptr;
  Target* d_tg = nullptr;
  uint32_t* d_flags = nullptr;
  uint32_t* d_ctl = nullptr;  // [0] epoch, [1] error
  std::vector<void*> bufs;
  std::vector<std::pair<int, int>> info;  // (R, S) per input product
};

__device__ __forceinline__ void swap32c(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// barrier that waits only for this wave's LDS operations (a compute wave's
// DMA stream stays in flight across it)
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 1 KB-per-instruction DMA copy global -> LDS (bytes % 16 == 0); the
// tail instruction is masked to the lanes that have data.
__device__ __forceinline__ void dma_copy(__amdgpu_buffer_rsrc_t r, uint32_t goff, uint32_t lds, int bytes,
                                         int lane) {
  for (int b = 0; b < bytes; b += 1024) {
    if (b + lane * 16 < bytes)
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 lds"
                   :: "v"(goff + (uint32_t)(b + lane * 16)), "s"(r), "s"(lds + (uint32_t)b) : "memory", "m0");
  }
}

// This wave's share of product q: tiles tfirst + t * tstep (t < tn), slice
// chunks [clo, chi), result slot part; valid only for an active workgroup.
struct Share {
  int tfirst, tstep, tn, clo, chi, part;
};

__device__ __forceinline__ Share share_of(const Op& o, int w, int v) {
  Share sh{0, 1, 0, 0, 0, 0};
  if (o.fmt == kFmtFin || w >= o.R * o.S) return sh;
  if (o.tiles_w >= kCW) {
    sh.tfirst = v;
    sh.tstep = kCW;
    sh.tn = (o.tiles_w - v + kCW - 1) / kCW;
    sh.clo = 0;
    sh.chi = o.chunks_w;
  } else {
    const int tile = v / o.wpt;
    if (tile >= o.tiles_w) return sh;
    sh.part = v - tile * o.wpt;
    sh.tfirst = tile;
    sh.tn = 1;
    sh.clo = sh.part * o.chunks_w / o.wpt;
    sh.chi = (sh.part + 1) * o.chunks_w / o.wpt;
  }
  return sh;
}

// Loading cursor of a compute wave over its chunk stream (all products in
// order); issue() enqueues the next chunk's two DMAs into ring slot `slot`.
struct Cursor {
  const Op* ops;
  int nops, w, v, lane;
  int q;
  Share sh;
  int t, c;
  // current product (buffer bases and sizes, made wave-uniform at each use)
  const void* cbase;
  const void* sbase;
  uint32_t cbytes, sbytes;
  uint32_t rowbytes, ngrp;
  int fmt, row0, chunk0;

  __device__ void enter(int qq) {
    for (q = __builtin_amdgcn_readfirstlane(qq); q < nops; ++q) {
      const Op& o = ops[__builtin_amdgcn_readfirstlane(q)];
      sh = share_of(o, w, v);
      if (sh.tn > 0 && sh.chi > sh.clo) {
        fmt = o.fmt;
        rowbytes = fmt == kFmtW4 ? (uint32_t)o.k / 2u : (uint32_t)o.k * 2u;
        ngrp = (uint32_t)o.k / 64u;
        cbase = o.codes;
        cbytes = (uint32_t)o.n * rowbytes;
        sbase = o.scales;
        sbytes = fmt == kFmtW4 ? (uint32_t)o.n * ngrp * 2u : 0u;
        const int r = w / o.S, s = w - r * o.S;
        row0 = r * o.rows;
        chunk0 = s * o.chunks_w;
        t = 0;
        c = sh.clo;
        return;
      }
    }
  }

  __device__ void issue(uint32_t slot_lds) {
    uint32_t coff = kOOB, soff = kOOB;
    const __amdgpu_buffer_rsrc_t r1 = rsrc(uniform_ptr(cbase), __builtin_amdgcn_readfirstlane(cbytes));
    const __amdgpu_buffer_rsrc_t r2 = rsrc(uniform_ptr(sbase), __builtin_amdgcn_readfirstlane(sbytes));
    if (q < nops) {
      const int tile = sh.tfirst + t * sh.tstep;
      const int j = lane & 15, kq = lane >> 4;
      const uint32_t row = (uint32_t)(row0 + tile * 16);
      const uint32_t gc = (uint32_t)(chunk0 + c);
      coff = (row + (uint32_t)j) * rowbytes + gc * 64u + (uint32_t)kq * 16u;
      if (fmt == kFmtW4) soff = ((row + (uint32_t)(lane >> 1)) * ngrp + 2u * gc + (uint32_t)(lane & 1)) * 2u;
      if (++c == sh.chi) {
        c = sh.clo;
        if (++t == sh.tn) enter(q + 1);
      }
    }
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :: "v"(coff), "s"(r1), "s"(slot_lds) : "memory", "m0");
    if (lane < 32)
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_ushort %0, %1, 0 offen lds"
                   :: "v"(soff), "s"(r2), "s"(slot_lds + (uint32_t)kSlotCode) : "memory", "m0");
  }
};

__device__ __forceinline__ bool poll_flags(const uint32_t* flags, int op, int wlo, int whi, uint32_t epoch,
                                           int lane, bool& dead, uint32_t* ctl) {
  if (dead) return false;
  const __amdgpu_buffer_rsrc_t rf = rsrc(flags + (size_t)op * kWG, kWG * 4);
  for (int it = 0; it < kSpinMax; ++it) {
    // agent scope (sc1) and volatile (bit 31): every poll reads memory again
    auto f = __builtin_amdgcn_raw_buffer_load_b128(rf, (uint32_t)lane * 16u, 0, (int)0x80000010u);
    asm volatile("" ::: "memory");
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane * 4 + i;
      ok = ok && (idx < wlo || idx >= whi || f[i] == epoch);
    }
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
  }
  if (lane == 0) {
    __hip_atomic_fetch_or(ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the first expiry: (op + 1) << 16 | producer range start << 8 | end - 1
    const uint32_t code = ((uint32_t)(op + 1) << 16) | ((uint32_t)wlo << 8) | (uint32_t)(whi - 1);
    uint32_t z = 0;
    __hip_atomic_compare_exchange_strong(ctl + 2, &z, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  dead = true;
  return false;
}

__global__ void __launch_bounds__(kThreads) chain_kernel(const Op* __restrict__ ops, int nops,
                                                         const Target* __restrict__ tg, uint32_t* flags,
                                                         uint32_t* ctl) {
  extern __shared__ uint4 lds4[];
  uint8_t* lds = (uint8_t*)lds4;
  uint8_t* stage = lds + kRingBytes;
  float* partl = (float*)(lds + kRingBytes + kStageBytes);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds4;
  const uint32_t stage_lds = lds_base + (uint32_t)kRingBytes;

  const int w = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool comm = wave == kCW;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, kq = lane >> 4;
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));

  // compute wave: its ring and loading cursor (the first kSlots chunks issued)
  const uint32_t ring = lds_base + (uint32_t)(wave * kSlots * kSlot);
  const uint8_t* ringp = lds + wave * kSlots * kSlot;
  Cursor cur;
  cur.ops = ops;
  cur.nops = nops;
  cur.w = w;
  cur.v = wave;
  cur.lane = lane;
  cur.cbase = nullptr;
  cur.sbase = nullptr;
  cur.cbytes = 0;
  cur.sbytes = 0;
  cur.q = nops;
  if (!comm) {
    cur.enter(0);
    for (int i = 0; i < kSlots; ++i) cur.issue(ring + (uint32_t)(i * kSlot));
  }
  int pos = 0;
  const uint16_t* xl = (const uint16_t*)stage;
  const int xb4 = (kq & 1) * 32 + (kq >> 1) * 16;  // int4 g64: this lane's k offset after the word exchange
  bool dead = false;

  for (int q = 0; q < nops; ++q) {
    const Op& o = ops[__builtin_amdgcn_readfirstlane(q)];
    const bool active = w < o.R * o.S;
    const int r = active ? w / o.S : 0, s = active ? w - r * o.S : 0;
    const int lo = s * o.kslice, L = o.kslice;
    const bool fin = o.fmt == kFmtFin;
    const bool reduce = active && !fin && !o.x_keep && o.src >= 0 && o.src_S > 1;

    // 1. the input slice: the communication wave waits for its producers and
    //    copies it (or their partials) into LDS
    if (comm) {
      if (fin) {
        // finalize the outputs no product consumed: rows [w*fr, (w+1)*fr) of
        // each target, in batches that fit the staging area
        int b0 = o.fin_lo;
        while (b0 < o.fin_hi) {
          int b1 = b0, used = 0;
          while (b1 < o.fin_hi) {
            const Target& t = tg[b1];
            const int fr = t.n / kWG;
            const int need = t.S * fr * 2;
            if (b1 > b0 && used + need > kStageBytes) break;
            const int rlo = w * fr / t.rows, rhi = ((w + 1) * fr - 1) / t.rows;
            poll_flags(flags, t.op, rlo * t.S, (rhi + 1) * t.S, epoch, lane, dead, ctl);
            const __amdgpu_buffer_rsrc_t rp = rsrc(t.part, (uint32_t)(t.S * t.n) * 2u);
            for (int sp = 0; sp < t.S; ++sp)
              dma_copy(rp, (uint32_t)(sp * t.n + w * fr) * 2u, stage_lds + (uint32_t)(used + sp * fr * 2), fr * 2,
                       lane);
            used += need;
            ++b1;
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          int off = 0;
          for (int b = b0; b < b1; ++b) {
            const Target& t = tg[b];
            const int fr = t.n / kWG;
            for (int e = lane * 8; e < fr; e += 512) {
              float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
              for (int sp = 0; sp < t.S; ++sp) {
                const half8 h = *(const half8*)(stage + off + sp * fr * 2 + e * 2);
#pragma unroll
                for (int i = 0; i < 8; ++i) a8[i] += (float)h[i];
              }
              half8 o8;
#pragma unroll
              for (int i = 0; i < 8; ++i) o8[i] = (_Float16)a8[i];
              *(half8*)(t.y + w * fr + e) = o8;
            }
            off += t.S * fr * 2;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          b0 = b1;
        }
      } else if (active && !o.x_keep) {
        if (o.src < 0) {
          dma_copy(rsrc(o.xext, (uint32_t)o.k * 2u), (uint32_t)lo * 2u, stage_lds, L * 2, lane);
        } else {
          const int rlo = lo / o.src_rows, rhi = (lo + L - 1) / o.src_rows;
          poll_flags(flags, o.src, rlo * o.src_S, (rhi + 1) * o.src_S, epoch, lane, dead, ctl);
          if (o.src_S == 1) {
            dma_copy(rsrc(o.src_y, (uint32_t)o.src_n * 2u), (uint32_t)lo * 2u, stage_lds, L * 2, lane);
          } else {
            const __amdgpu_buffer_rsrc_t rp = rsrc(o.src_part, (uint32_t)(o.src_S * o.src_n) * 2u);
            for (int sp = 0; sp < o.src_S; ++sp)
              dma_copy(rp, (uint32_t)(sp * o.src_n + lo) * 2u, stage_lds + (uint32_t)(sp * L * 2), L * 2, lane);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
    bar();  // A: copies in LDS

    // 2. every wave adds partials: element e of the slice is the fp32 sum of
    //    the src_S partials in slice order, rounded once to fp16, written over
    //    the first partial
    if (reduce) {
      for (int e = (int)threadIdx.x * 8; e < L; e += kThreads * 8) {
        float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < o.src_S; ++sp) {
          const half8 h = *(const half8*)(stage + (sp * L + e) * 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) a8[i] += (float)h[i];
        }
        half8 o8;
#pragma unroll
        for (int i = 0; i < 8; ++i) o8[i] = (_Float16)a8[i];
        *(half8*)(stage + e * 2) = o8;
      }
    }
    bar();  // B: input slice ready

    if (!comm) {
      // 3. this wave's share: chunk by chunk from the ring
      const Share sh = share_of(o, w, wave);
      if (sh.chi > sh.clo) {
        for (int t = 0; t < sh.tn; ++t) {
          const int tile = sh.tfirst + t * sh.tstep;
          float acc = 0.f;
          if (o.fmt == kFmtW4) {
            for (int c = sh.clo; c < sh.chi; ++c) {
              asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * (kSlots - 1)) : "memory");
              const uint8_t* sl = ringp + pos * kSlot;
              const uint4 c4 = *(const uint4*)(sl + lane * 16);
              const uint2 s2 = *(const uint2*)(sl + kSlotCode + 8 * j);
              uint32_t w0 = c4.x, w1 = c4.y, w2 = c4.z, w3 = c4.w;
              swap32c(w0, w2);
              swap32c(w1, w3);
              const uint16_t* xp = xl + c * 128 + xb4;
              half8 a0 = {0, 0, 0, 0, 0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
              if (j == 0) {
                a0 = *(const half8*)(xp);
                a1 = *(const half8*)(xp + 8);
                a2 = *(const half8*)(xp + 64);
                a3 = *(const half8*)(xp + 72);
              }
              const float4v z = {0.f, 0.f, 0.f, 0.f};
              float4v g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, dec4n<true>(w0), z, 0, 0, 0);
              g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, dec4n<true>(w1), g0, 0, 0, 0);
              float4v g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, dec4n<true>(w2), z, 0, 0, 0);
              g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, dec4n<true>(w3), g1, 0, 0, 0);
              const float sc0 = f16_bits_to_f32((uint16_t)(s2.x & 0xffffu));
              const float sc1 = f16_bits_to_f32((uint16_t)(s2.y & 0xffffu));
              acc += sc0 * g0[0];
              acc += sc1 * g1[0];
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before it is refilled
              cur.issue(ring + (uint32_t)(pos * kSlot));
              pos = pos + 1 == kSlots ? 0 : pos + 1;
            }
          } else {
            float4v acc4 = {0.f, 0.f, 0.f, 0.f};
            for (int c = sh.clo; c < sh.chi; ++c) {
              asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * (kSlots - 1)) : "memory");
              const uint8_t* sl = ringp + pos * kSlot;
              const half8 b = __builtin_bit_cast(half8, *(const uint4*)(sl + lane * 16));
              half8 a = {0, 0, 0, 0, 0, 0, 0, 0};
              if (j == 0) a = *(const half8*)(xl + c * 32 + 8 * kq);
              acc4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc4, 0, 0, 0);
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              cur.issue(ring + (uint32_t)(pos * kSlot));
              pos = pos + 1 == kSlots ? 0 : pos + 1;
            }
            acc = acc4[0];
          }
          if (lane < 16) partl[(tile * o.wpt + sh.part) * 16 + j] = acc;
        }
      }
    } else if (o.fin_src && active && !fin && !o.x_keep && r == 0) {
      // the first consumer's row-block-0 workgroups store the reduced input
      // as the producer's output
      for (int e = lane * 8; e < L; e += 512) *(uint4*)(o.src_y + lo + e) = *(const uint4*)(stage + e * 2);
    }
    bar();  // C: results in LDS

    // 4. the communication wave sums each tile's K parts, stores the results
    //    (fp16 output, or this slice's fp16 partial), waits for the stores and
    //    publishes the flag
    if (comm && active && !fin) {
      uint16_t* dst = o.S == 1 ? o.y : o.part + (size_t)s * o.n;
      const __amdgpu_buffer_rsrc_t rd = rsrc(dst, (uint32_t)o.n * 2u);
      for (int e = lane * 8; e < o.rows; e += 512) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = e + 2 * i + h, tile = row >> 4, jj = row & 15;
            float v = 0.f;
            for (int p = 0; p < o.wpt; ++p) v += partl[(tile * o.wpt + p) * 16 + jj];
            v2[h] = v;
          }
          pk[i] = (uint32_t)f32_to_f16_bits(v2[0]) | ((uint32_t)f32_to_f16_bits(v2[1]) << 16);
        }
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 val = {pk[0], pk[1], pk[2], pk[3]};
        __builtin_amdgcn_raw_buffer_store_b128(val, rd, (uint32_t)(r * o.rows + e) * 2u, 0, 16);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0)
        __hip_atomic_store(flags + (size_t)q * kWG + w, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// the next launch's epoch (never 0, the value of fresh flags)
__global__ void chain_epoch_kernel(uint32_t* ctl) {
  const uint32_t e = ctl[0] + 1u;
  ctl[0] = e == 0u ? 1u : e;
}

}  // namespace

// ---------------------------------------------------------------------------
// host: planning, plan memory, launch
// ---------------------------------------------------------------------------

// Choose each product's R x S grid.  Preference: S = 16 with R = 16 (each
// consumer then waits for about 16 producers), then other splits; a product
// that shares its predecessor's input keeps that grid so the input slice
// stays in LDS.  Limits: rows a multiple of 16, slices a multiple of the
// chunk, at most 64 tile parts per workgroup, an input slice of at most
// 16384 values, partial staging within 32 KB, buffers below 2 GiB.
static bool plan_op(const ChainOpIn* in, int nin, const std::vector<Op>& done, int q, Op& o) {
  const ChainOpIn& a = in[q];
  // an output that no later product reads is finalized by the last pass,
  // which takes n / 256 rows per workgroup in 8-row multiples
  bool consumed = false;
  for (int p = q + 1; p < nin; ++p) consumed = consumed || in[p].src == q;
  const int ck = a.fmt == kFmtW4 ? 128 : 32;
  const int srcS = a.src >= 0 ? done[a.src].S : 1;
  auto fits = [&](int R, int S) -> bool {
    if (R < 1 || S < 1 || R * S > kWG) return false;
    if (a.n % (R * 16) != 0 || a.k % (S * ck) != 0) return false;
    const int rows = a.n / R, tiles = rows / 16, chunks = a.k / S / ck;
    const int wpt = tiles >= kCW ? 1 : (kCW / tiles < chunks ? kCW / tiles : chunks);
    if (tiles * wpt > kPartBytes / 64) return false;
    const int L = a.k / S;
    if (L > kStageBytes / 2) return false;
    if (a.src >= 0 && srcS > 1 && srcS * L * 2 > kStageBytes) return false;
    if (S > 1 && !consumed && (a.n % (kWG * 8) != 0 || S * (a.n / kWG) * 2 > kStageBytes)) return false;
    return true;
  };
  auto take = [&](int R, int S) {
    o.R = R;
    o.S = S;
    o.rows = a.n / R;
    o.kslice = a.k / S;
    o.tiles_w = o.rows / 16;
    o.chunks_w = o.kslice / ck;
    o.wpt = o.tiles_w >= kCW ? 1 : (kCW / o.tiles_w < o.chunks_w ? kCW / o.tiles_w : o.chunks_w);
  };
  if (q > 0) {
    const Op& p = done[q - 1];
    if (p.fmt != kFmtFin && in[q - 1].src == a.src && in[q - 1].k == a.k && fits(p.R, p.S)) {
      take(p.R, p.S);
      o.x_keep = 1;
      return true;
    }
  }
  static const int pref[] = {16, 8, 32, 4, 64, 2, 128, 1, 256};
  for (int S : pref) {
    for (int R = kWG / S; R >= 1; R >>= 1) {
      if (fits(R, S)) {
        take(R, S);
        return true;
      }
    }
  }
  return false;
}

int chain_create(const ChainOpIn* in, int nin, void** out) {
  *out = nullptr;
  if (nin < 1) return -2;
  std::vector<Op> ops(nin);
  for (int q = 0; q < nin; ++q) {
    const ChainOpIn& a = in[q];
    Op& o = ops[q];
    memset(&o, 0, sizeof(o));
    if (a.fmt != kFmtW4 && a.fmt != kFmtF16) return -4;
    if (a.src >= q || a.src < -1) return -2;
    if (a.src >= 0 && in[a.src].n != a.k) return -2;
    if (a.src < 0 && !a.x) return -1;
    if (!a.codes || !a.y || (a.fmt == kFmtW4 && !a.scales)) return -1;
    const size_t rowbytes = a.fmt == kFmtW4 ? (size_t)a.k / 2 : (size_t)a.k * 2;
    if ((size_t)a.n * rowbytes >= ((size_t)1 << 31)) return -2;
    o.codes = (const uint8_t*)a.codes;
    o.scales = a.scales;
    o.y = a.y;
    o.xext = a.x;
    o.fmt = a.fmt;
    o.n = a.n;
    o.k = a.k;
    o.src = a.src;
    if (!plan_op(in, nin, ops, q, o)) return -2;
    if (a.src >= 0) {
      const Op& p = ops[a.src];
      o.src_S = p.S;
      o.src_rows = p.rows;
      o.src_n = p.n;
      o.src_y = p.y;
    }
  }
  // outputs with partials: the first consumer finalizes them; the others go
  // to FIN, which needs 8-row multiples per workgroup (else the product is
  // re-planned unsplit... which the planner above cannot do after the fact:
  // such shapes are refused)
  std::vector<int> fin_targets;
  for (int q = 0; q < nin; ++q) {
    if (ops[q].S == 1) continue;
    int c = -1;
    for (int p = q + 1; p < nin && c < 0; ++p)
      if (in[p].src == q && !ops[p].x_keep) c = p;
    if (c >= 0) {
      ops[c].fin_src = 1;
    } else {
      if (ops[q].n % (kWG * 8) != 0) return -2;
      if (ops[q].S * (ops[q].n / kWG) * 2 > kStageBytes) return -2;
      fin_targets.push_back(q);
    }
  }
  Plan* pl = new Plan();
  auto fail = [&](hipError_t e) {
    for (void* b : pl->bufs) hipFree(b);
    delete pl;
    return e == hipSuccess ? -2 : -7;
  };
  auto alloc = [&](size_t bytes, void** p) -> hipError_t {
    hipError_t e = hipMalloc(p, bytes);
    if (e == hipSuccess) pl->bufs.push_back(*p);
    return e;
  };
  hipError_t e;
  for (int q = 0; q < nin; ++q) {
    if (ops[q].S > 1) {
      void* p = nullptr;
      if ((e = alloc((size_t)ops[q].S * ops[q].n * 2, &p)) != hipSuccess) return fail(e);
      ops[q].part = (uint16_t*)p;
    }
  }
  for (int q = 0; q < nin; ++q)
    if (ops[q].src >= 0) ops[q].src_part = ops[ops[q].src].part;
  std::vector<Target> tg;
  for (int q : fin_targets) tg.push_back(Target{ops[q].y, ops[q].part, q, ops[q].n, ops[q].S, ops[q].rows});
  if (!tg.empty()) {
    Op f;
    memset(&f, 0, sizeof(f));
    f.fmt = kFmtFin;
    f.R = 1;
    f.S = 1;
    f.src = -1;
    f.fin_lo = 0;
    f.fin_hi = (int)tg.size();
    ops.push_back(f);
  }
  pl->nops = (int)ops.size();
  void *dops = nullptr, *dtg = nullptr, *dflags = nullptr, *dctl = nullptr;
  if ((e = alloc(ops.size() * sizeof(Op), &dops)) != hipSuccess) return fail(e);
  if ((e = alloc((tg.size() + 1) * sizeof(Target), &dtg)) != hipSuccess) return fail(e);
  if ((e = alloc(ops.size() * kWG * 4, &dflags)) != hipSuccess) return fail(e);
  if ((e = alloc(16, &dctl)) != hipSuccess) return fail(e);
  const uint32_t ctl0[4] = {1u, 0u, 0u, 0u};
  if ((e = hipMemcpy(dops, ops.data(), ops.size() * sizeof(Op), hipMemcpyHostToDevice)) != hipSuccess) return fail(e);
  if (!tg.empty() &&
      (e = hipMemcpy(dtg, tg.data(), tg.size() * sizeof(Target), hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e);
  if ((e = hipMemset(dflags, 0, ops.size() * kWG * 4)) != hipSuccess) return fail(e);
  if ((e = hipMemcpy(dctl, ctl0, sizeof(ctl0), hipMemcpyHostToDevice)) != hipSuccess) return fail(e);
  static bool attr = false;
  if (!attr) {
    if ((e = hipFuncSetAttribute((const void*)chain_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes)) !=
        hipSuccess)
      return fail(e);
    attr = true;
  }
  int dev = 0, cus = 0, per = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return fail(e);
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return fail(e);
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)chain_kernel, kThreads, kLdsBytes)) !=
      hipSuccess)
    return fail(e);
  // every workgroup must be resident at once
  if (per < 1 || cus * per < kWG) return fail(hipSuccess);
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e);
  pl->d_ops = (Op*)dops;
  pl->d_tg = (Target*)dtg;
  pl->d_flags = (uint32_t*)dflags;
  pl->d_ctl = (uint32_t*)dctl;
  pl->info.resize(nin);
  for (int q = 0; q < nin; ++q) pl->info[q] = {ops[q].R, ops[q].S};
  *out = pl;
  return 0;
}

hipError_t chain_run(void* plan, hipStream_t st) {
  Plan* pl = (Plan*)plan;
  hipLaunchKernelGGL(chain_kernel, dim3(kWG), dim3(kThreads), kLdsBytes, st, (const Op*)pl->d_ops, pl->nops,
                     (const Target*)pl->d_tg, pl->d_flags, pl->d_ctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_epoch_kernel, dim3(1), dim3(1), 0, st, pl->d_ctl);
  return hipGetLastError();
}

int chain_error(void* plan, uint32_t* err) {
  Plan* pl = (Plan*)plan;
  uint32_t ctl[4] = {0, 0, 0, 0};
  if (hipDeviceSynchronize() != hipSuccess) return -7;
  if (hipMemcpy(ctl, pl->d_ctl, sizeof(ctl), hipMemcpyDeviceToHost) != hipSuccess) return -7;
  err[0] = ctl[1];
  err[1] = ctl[2];
  err[2] = ctl[0];
  return 0;
}

int chain_grid(void* plan, int q, int* R, int* S) {
  Plan* pl = (Plan*)plan;
  if (q < 0 || q >= (int)pl->info.size()) return -2;
  *R = pl->info[q].first;
  *S = pl->info[q].second;
  return 0;
}

void chain_destroy(void* plan) {
  Plan* pl = (Plan*)plan;
  if (!pl) return;
  hipDeviceSynchronize();
  for (void* b : pl->bufs) hipFree(b);
  delete pl;
}

}  // namespace rq
