// kernels.h -- gfx950 kernels of the boundary path (included by the k_*.hip
// translation units, which instantiate them per source kind).
//
// One workgroup per token row. The row is split into 16-byte vectors of 8
// elements; thread t of a workgroup of `threads` lanes owns vectors
// t, t + threads, ... (VPT of them), so each load instruction of a wavefront
// reads 1 KiB of contiguous row. Two families of kernels, chosen per launch
// by the host: read_kernel and complete_kernel give a row several wavefronts
// and issue all of its loads before any arithmetic; wave_read_kernel and
// wave_complete_kernel give a row one wavefront that streams the sources one
// after another with two loads in flight. The row's work:
//   1. complete: load the sources (P partials, or the k gathered expert rows)
//      and the residual and sum them in fp32 in source order (the deferred
//      all-reduce of the study note's fusion point, on one GPU a sum over
//      resident buffers);
//   2. fold: x = r + s in fp32 (guide, "Residual update and input read": the
//      plain update is an add and the read keeps the fp32 sum);
//   3. read: sum of squares over the row in one order whatever the launch
//      shape (per vector, then per lane in vector order, then a wave64 DPP
//      sum; see row_reduce), inv = 1/sqrt(ss/H + eps) (correctly rounded
//      divide and square root), y = (x * w) * inv;
//   4. store the residual as bf16 (round to nearest even, v_cvt_pk_bf16_f32)
//      and y as bf16, or as OCP e4m3 codes (v_cvt_pk_fp8_f32) with a
//      per-row fp32 scale.
// No atomics: the result is bitwise reproducible run to run, and the same for
// every launch shape.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <atomic>
#include <type_traits>
#include <utility>

#include "launch.h"

namespace bnd {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Row access through buffer resources. Every row operand gets a resource whose
// base is the row and whose size is the row's bytes, so each access is
// bounds-checked by the hardware (an out-of-range load returns 0 and an
// out-of-range store is dropped); read_kernel also guards its stores by lane,
// the one-wavefront read relies on the resource alone.
// Cache policy: rows are read exactly once, so loads are non-temporal (nt);
// stores carry sc1 (write-through past the XCD's L2). Both measured faster on
// MI355X than the default policy for this 9:2 read:write stream. The
// multi-wave reads with one vector per thread are also built with
// non-temporal stores, which the host takes for launches of fewer rows than
// CUs (decode boundaries): 3% faster there, and 3-3.6% slower on launches of
// one row per CU and more.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit data format, raw addressing
constexpr int kLoadOnce = 2;            // cache policy bits: nt
constexpr int kStoreStream = 16;        // cache policy bits: sc1
constexpr int kStoreOnce = 2;           // cache policy bits: nt

__device__ __forceinline__ Rsrc row_rsrc(const void* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 load16(Rsrc r, int byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kLoadOnce);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int kPolicy = kStoreStream>
__device__ __forceinline__ void store16(Rsrc r, int byte_off, uint4 v) {
  const u32x4 u = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, byte_off, 0, kPolicy);
}

template <int kPolicy = kStoreStream>
__device__ __forceinline__ void store8(Rsrc r, int byte_off, uint2 v) {
  const u32x2 u = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(u, r, byte_off, 0, kPolicy);
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float f[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

// Two floats -> two bf16 (round to nearest even), low element first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint4 f32_to_bf16x8(const float f[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Eight floats (already within +-448) -> eight OCP e4m3 codes, element 0 in
// the lowest byte.
__device__ __forceinline__ uint2 f32_to_e4m3x8(const float f[8]) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// The e4m3 inputs of eight y values of a row: the fp32 quotient y / scale,
// correctly rounded, clamped to +-448. `rcp` is the correctly rounded 1 /
// scale (one division per row); q = y * rcp is then within one ulp of
// y / scale, r = y - q * scale is exact as one fma, and q + r * rcp as one
// fma is the correctly rounded quotient (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990), so a code is decided on the same fp32 value a division
// gives, midpoints included. A zero scale (a zero row) has rcp = 0 and gives
// +0 codes. A scale below 2^-128, which only a row of tiny (subnormal)
// weights reaches, has no finite reciprocal: such a row takes kDivide, since
// y * inf would give +-448 for small y and NaN for y = 0.
template <bool kDivide>
__device__ __forceinline__ void fp8_inputs(const float (&y)[8], float scale, float rcp, float (&t)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float q;
    if constexpr (kDivide) {
      q = y[e] / scale;
    } else {
      q = y[e] * rcp;
      q = fmaf(fmaf(-q, scale, y[e]), rcp, q);
    }
    t[e] = fminf(fmaxf(q, -448.0f), 448.0f);
  }
}

__device__ __forceinline__ bool fp8_divide(float rcp) { return !(rcp <= 3.40282347e38f); }

// ---------------------------------------------------------------------------
// wave64 reductions (DPP). Lanes are in four rows of 16: a butterfly inside
// each row (quad_perm, half-mirror, mirror), then row_bcast:15 / row_bcast:31
// carry the row results upward so lane 63 holds the wave's total.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadSwap1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadSwap2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppQuadSwap1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppQuadSwap2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppRowHalfMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppRowMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, kDppRowBcast31, 0xC, 0xF, false);
  return lane63(v);
}

// max of non-negative values (0 is the identity)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppQuadSwap1, 0xF, 0xF, false));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppQuadSwap2, 0xF, 0xF, false));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppRowHalfMirror, 0xF, 0xF, false));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppRowMirror, 0xF, 0xF, false));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppRowBcast15, 0xA, 0xF, false));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, kDppRowBcast31, 0xC, 0xF, false));
  return lane63(v);
}

// The sum of squares of a row, in one order that does not depend on the launch
// shape, so that a row gets the same inv (and so the same y and fp8 codes) from
// every kernel and workgroup size, in a full call and in a share of its rows:
//   q_v  = the squares of vector v's eight elements added in element order,
//          one fma each, from 0 (vector_ss);
//   A_l  = q_l + q_{l+64} + q_{l+128} + ..., added left to right, for each of
//          the 64 lanes l (the vectors a lane of a one-wavefront row owns, in
//          the order it owns them);
//   sum  = wave_sum over the 64 A_l.
// Vectors past the end of the row count as q = +0, which leaves every sum
// unchanged, so the number of lanes and vectors a launch has beyond the row
// does not matter either.
__device__ __forceinline__ float vector_ss(const float (&x)[8]) {
  float q = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) q = fmaf(x[e], x[e], q);
  return q;
}

// The row's total from a workgroup of blockDim.x threads (a multiple of 64),
// thread t holding the q of vectors t, t + blockDim.x, ... (VPT of them): with
// several wavefronts every q goes to LDS by its vector index and, after one
// barrier, every lane l adds the q of vectors l, l + 64, ... in that order and
// the wavefront sums the 64 lane totals, so all threads hold the same result.
// With kWithMax the row's max of mx (non-negative values) too, through one LDS
// slot per wave (a max does not depend on its order).
template <int VPT, bool kWithMax>
__device__ __forceinline__ void row_reduce(const float (&q)[VPT], float& ss, float& mx, float* lds_q,
                                           float* lds_max) {
  const int nthr = blockDim.x;
  const int nw = nthr / kWave;
  const int tid = threadIdx.x;
  float lane_total = 0.0f;
  if (nw == 1) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) lane_total += q[v];
    ss = wave_sum(lane_total);
    if constexpr (kWithMax) mx = wave_max(mx);
    return;
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) lds_q[tid + v * nthr] = q[v];
  if constexpr (kWithMax) {
    mx = wave_max(mx);
    if ((tid % kWave) == 0) lds_max[tid / kWave] = mx;
  }
  __syncthreads();
  const int lane = tid % kWave;
  const int n = nw * VPT;  // vectors per lane l: l, l + 64, ..., l + 64 (n - 1)
  for (int j = 0; j < n; ++j) lane_total += lds_q[lane + j * kWave];
  ss = wave_sum(lane_total);
  if constexpr (kWithMax) {
    float m = 0.0f;
    for (int i = 0; i < nw; ++i) m = fmaxf(m, lds_max[i]);
    mx = m;
  }
}

// ---------------------------------------------------------------------------
// Loading and completing the contribution of one row: x[v][e] for the
// thread's VPT vectors. Lanes past the end of the row hold zeros.
// ---------------------------------------------------------------------------

// A MoE row's picks: lane j < k holds the index and gate of pick j, fetched
// with one load each when the row starts (lanes >= k read 0 through the
// resource's bounds), so resolving a pick later is a register read
// (v_readlane), not a dependent memory access, and no load waits on another:
// a dropped pick's gate is replaced by 0 after both loads have returned.
struct RowPicks {
  int idx = 0;
  float gate = 0.0f;
};

__device__ __forceinline__ RowPicks load_picks(const RowArgs& a, int64_t row, int k, int lane) {
  const Rsrc ir = row_rsrc(a.idx + row * k, k * 4);
  const Rsrc gr = row_rsrc(a.gate + row * k, k * 4);
  RowPicks p;
  p.idx = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, lane * 4, 0, 0);
  p.gate = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, lane * 4, 0, 0));
  return p;
}

// Pick j of a row (wave-uniform): its expert row, -1 when the index is outside
// the buffer, and its gate, 0 for such a dropped pick whatever the gate holds.
__device__ __forceinline__ void resolve_pick(const RowArgs& a, const RowPicks& picks, int j, int64_t& er, float& g) {
  const int64_t e = __builtin_amdgcn_readlane(picks.idx, j);
  const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(picks.gate), j));
  const bool valid = e >= 0 && e < a.n_expert_rows;
  er = valid ? e : -1;
  g = valid ? gj : 0.0f;
}

// Loads are issued by every lane without a guard: a lane past the end of the
// row addresses beyond its row resource and reads 0, which keeps the loads
// branch-free so they can all be in flight together.
//
// Keeps a step's arithmetic at its place in the pipeline: the empty asm reads
// and writes the eight sums, so they are computed before it, and the
// scheduling fence after it keeps later loads behind it. (A fence alone does
// not stop the compiler from sinking the adds towards their later uses.)
__device__ __forceinline__ void pin8(float (&x)[8]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
}

// Vectors whose source loads are in flight together. A batch of kb vectors
// holds 4*(N+1)*kb VGPRs of raw loads next to the row's fp32 values and
// weights (16*VPT) and `per_source` more for each source's bookkeeping (two
// for a MoE pick); the largest kb <= VPT that keeps the estimate within the
// 128 VGPRs of a 1024-thread workgroup avoids scratch spills. Each finished
// batch's sums are pinned in place before the next batch's loads: otherwise
// the compiler sinks them towards the stores and every batch's raw loads stay
// live together (a 16-source snapshot with four vectors per thread spilled
// 636 bytes per lane that way).
constexpr int load_batch(int n, int vpt, int per_source = 0) {
  for (int kb = vpt; kb > 1; kb /= 2)
    if (4 * (n + 1) * kb + 16 * vpt + 12 + per_source * n <= 128) return kb;
  return 1;
}
// kFold = false computes the contribution s alone (complete_only). kPolicy is
// the cache policy of the enter's copy of the input into the residual.
template <Source S, int N, int VPT, bool kFold = true, int kPolicy = kStoreStream>
__device__ __forceinline__ void load_and_fold(const RowArgs& a, int64_t row, int tid, int nthr,
                                              const bool (&ok)[VPT], float (&x)[VPT][8]) {
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const int row_bytes = a.H * 2;
  int off[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) off[v] = (tid + v * nthr) * 16;
  const Rsrc res = row_rsrc(a.res + row * a.ld_res, row_bytes);
  // the residual as a fold input: an empty resource (loads read 0) when the
  // stream is Pending without a residual
  const Rsrc res_in = row_rsrc(a.res + row * a.ld_res, a.has_residual ? row_bytes : 0);
  if constexpr (S == Source::Partials) {
    constexpr int kB = load_batch(N, VPT);
#pragma unroll
    for (int v0 = 0; v0 < VPT; v0 += kB) {
      uint4 c[N][kB];
      uint4 r[kB];
#pragma unroll
      for (int p = 0; p < N; ++p) {
        const Rsrc src = row_rsrc(a.src[p] + row * a.ld_src, row_bytes);
#pragma unroll
        for (int b = 0; b < kB; ++b) c[p][b] = load16(src, off[v0 + b]);
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) r[b] = kFold ? load16(res_in, off[v0 + b]) : zero;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        float s[8], t[8], rv[8];
        bf16x8_to_f32(c[0][b], s);
#pragma unroll
        for (int p = 1; p < N; ++p) {
          bf16x8_to_f32(c[p][b], t);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] += t[e];
        }
        bf16x8_to_f32(r[b], rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[v0 + b][e] = rv[e] + s[e];
        if constexpr (kB < VPT) pin8(x[v0 + b]);
      }
      // keep the next batch's loads behind this batch's sums (register budget)
      if constexpr (kB < VPT) __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (S == Source::Moe) {
    // A dropped pick (index outside the expert rows) reads zeros through an empty resource and
    // its product is not added, so it contributes nothing whatever its gate holds (NaN or inf
    // too). The choice is made on the sum, not on the loaded gate: a select on a loaded value
    // may be compiled as a branch around the load, one memory round trip per pick.
    int64_t er[N];
    float g[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int64_t e = a.idx[row * N + j];
      const bool valid = e >= 0 && e < a.n_expert_rows;
      er[j] = valid ? e : -1;
      g[j] = a.gate[row * N + j];
    }
    constexpr int kB = load_batch(N, VPT, 2);
#pragma unroll
    for (int v0 = 0; v0 < VPT; v0 += kB) {
      uint4 c[N][kB];
      uint4 r[kB];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        // an invalid pick gets an empty resource: its loads return 0 and its product is dropped
        const Rsrc src = row_rsrc(a.experts + (er[j] < 0 ? 0 : er[j]) * a.ld_e, er[j] < 0 ? 0 : row_bytes);
#pragma unroll
        for (int b = 0; b < kB; ++b) c[j][b] = load16(src, off[v0 + b]);
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) r[b] = kFold ? load16(res_in, off[v0 + b]) : zero;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        float s[8], t[8], rv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
          bf16x8_to_f32(c[j][b], t);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = er[j] >= 0 ? fmaf(g[j], t[e], s[e]) : s[e];
        }
        bf16x8_to_f32(r[b], rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[v0 + b][e] = rv[e] + s[e];
        if constexpr (kB < VPT) pin8(x[v0 + b]);
      }
      // keep the next batch's loads behind this batch's sums (register budget)
      if constexpr (kB < VPT) __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // Input: the stack input x_in (enter); Residual: the stored residual (written read)
    const Rsrc src = (S == Source::Input) ? row_rsrc(a.x_in + row * a.ld_x, row_bytes) : res;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const uint4 raw = load16(src, off[v]);
      if constexpr (S == Source::Input) {
        if (ok[v] && a.copy_input) store16<kPolicy>(res, off[v], raw);
      }
      bf16x8_to_f32(raw, x[v]);
    }
  }
}

template <int VPT>
__device__ __forceinline__ void load_weight(const RowArgs& a, int tid, int nthr, float (&w)[VPT][8]) {
  // the weight is shared by all rows: default cache policy, it stays in L2
  const Rsrc wr = row_rsrc(a.w, a.H * 4);
  // Gemma form: the stored weight is an offset from one. Added without a branch (w + 0 for the
  // plain form) so the weight loads schedule like the rest of the row's loads.
  const float offset = a.gemma ? 1.0f : 0.0f;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int off = (tid + v * nthr) * 32;
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(wr, off + 16, 0, 0);
    w[v][0] = __uint_as_float(lo.x) + offset; w[v][1] = __uint_as_float(lo.y) + offset;
    w[v][2] = __uint_as_float(lo.z) + offset; w[v][3] = __uint_as_float(lo.w) + offset;
    w[v][4] = __uint_as_float(hi.x) + offset; w[v][5] = __uint_as_float(hi.y) + offset;
    w[v][6] = __uint_as_float(hi.z) + offset; w[v][7] = __uint_as_float(hi.w) + offset;
  }
}

// ---------------------------------------------------------------------------
// The boundary read kernel: complete, fold, RMSNorm, stores.
// ---------------------------------------------------------------------------
// kNt: non-temporal stores (launches of fewer rows than CUs), else sc1.
template <Source S, int N, int VPT, bool FP8, bool kNt = false>
__global__ __launch_bounds__(kMaxThreads) void read_kernel(const RowArgs a) {
  constexpr int kPol = kNt ? kStoreOnce : kStoreStream;
  __shared__ float lds_q[kMaxThreads * VPT];  // the row's per-vector sums of squares, by vector
  __shared__ float lds_max[kMaxThreads / kWave];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  bool ok[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) ok[v] = (tid + v * nthr) < a.nvec;

  float x[VPT][8];
  load_and_fold<S, N, VPT, true, kPol>(a, row, tid, nthr, ok, x);
  // with four vectors per thread the weights wait until the loads are summed
  if constexpr (VPT >= 4) __builtin_amdgcn_sched_barrier(0);
  float w[VPT][8];
  load_weight<VPT>(a, tid, nthr, w);

  float ss = 0.0f, mx = 0.0f, q[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) q[v] = vector_ss(x[v]);
  if constexpr (FP8) {
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[v][e] * w[v][e]));
  }
  row_reduce<VPT, FP8>(q, ss, mx, lds_q, lds_max);
  const float inv = 1.0f / sqrtf(ss / (float)a.H + a.eps);

  const int row_bytes = a.H * 2;
  if constexpr (S == Source::Partials || S == Source::Moe) {
    const Rsrc res = row_rsrc(a.res + row * a.ld_res, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
      if (ok[v]) store16<kPol>(res, (tid + v * nthr) * 16, f32_to_bf16x8(x[v]));
  }

  if constexpr (!FP8) {
    const Rsrc yr = row_rsrc(a.y + row * a.ld_y, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (x[v][e] * w[v][e]) * inv;  // the one-wavefront read's order
      if (ok[v]) store16<kPol>(yr, (tid + v * nthr) * 16, f32_to_bf16x8(y));
    }
  } else {
    // y_h = (x_h w_h) inv. Rounding is monotone, so max_h |y_h| is exactly
    // (max_h |x_h w_h|) inv: the scale is fp32(max|y| / 448) of these y.
    const float amax = mx * inv;
    const float scale = amax / 448.0f;
    const float rcp = scale > 0.0f ? 1.0f / scale : 0.0f;
    const Rsrc qr = row_rsrc(a.q + row * a.ld_q, a.H);
    const auto codes = [&](auto divide) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float y[8], t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (x[v][e] * w[v][e]) * inv;
        fp8_inputs<decltype(divide)::value>(y, scale, rcp, t);
        if (ok[v]) store8<kPol>(qr, (tid + v * nthr) * 8, f32_to_e4m3x8(t));
      }
    };
    if (fp8_divide(rcp))  // uniform across the row
      codes(std::true_type{});
    else
      codes(std::false_type{});
    if (tid == 0) a.scale[row] = scale;
  }
}

// complete_only / add_to_output (kFold = false): the contribution, plus the
// extra row when one is given, stored as bf16. snapshot (kFold = true): the
// folded row r + s stored as bf16 into a separate output; the residual is
// only read.
template <Source S, int N, int VPT, bool kFold>
__global__ __launch_bounds__(kMaxThreads) void complete_kernel(const RowArgs a) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  bool ok[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) ok[v] = (tid + v * nthr) < a.nvec;
  float s[VPT][8];
  load_and_fold<S, N, VPT, kFold>(a, row, tid, nthr, ok, s);
  if constexpr (!kFold) {
    if (a.extra) {
      const Rsrc ex = row_rsrc(a.extra + row * a.ld_extra, a.H * 2);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float t[8];
        bf16x8_to_f32(load16(ex, (tid + v * nthr) * 16), t);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[v][e] += t[e];
      }
    }
  }
  const Rsrc out = row_rsrc(a.y + row * a.ld_y, a.H * 2);
#pragma unroll
  for (int v = 0; v < VPT; ++v)
    if (ok[v]) store16(out, (tid + v * nthr) * 16, f32_to_bf16x8(s[v]));
}

// ---------------------------------------------------------------------------
// The boundary read with one wavefront per row, for folds of partials or MoE
// picks: 64 lanes x VPT vectors, VPT an even count from 2 (rows of up to 1024
// elements) to 14 (up to 7168); 51..255 VGPRs, two to eight waves per SIMD.
//
// Used from 6 rows per CU (12 at the width of 2) when a launch's rows fill
// their rounds of resident rows well (on 256 CUs: the 2048-row prefill,
// quantised and MoE boundaries).
// What makes it faster there than the multi-wave rows of read_kernel, all
// measured on MI355X:
//  - loads go source by source (every vector of source 0, then of source 1,
//    ..., the residual last), so a wave streams one contiguous row of one
//    operand at a time; vector-major order is up to 25% slower;
//  - two loads are kept in flight per wave through a two-register ring (one
//    in flight is latency-bound, more is slower);
//  - each vector is finished during the residual pass, so nothing but a few
//    multiplies and the stores follow the row's reduction: the residual is
//    stored at once, x^2 and |x w| are accumulated, and only x w is kept (the
//    weight vector is loaded together with the residual's). The row then
//    holds one set of 8 * VPT floats, not x and w both. Loading the weight
//    after the reduction, or quantising with a full division per element,
//    leaves HBM idle at the tail of the single round (7% and 10% slower).
// The reduction is a wavefront DPP sum with no LDS and no barrier. The sum of
// the sources runs in the same order per element as in load_and_fold, so the
// residual is bitwise the same as with read_kernel; y = (x w) inv, and the
// fp8 codes are those of (x w) inv times the reciprocal of the row's scale.
// ---------------------------------------------------------------------------
// Loads each wave keeps in flight through its ring by default, per width: a
// divisor of the width, so that the ring slot of a load is its vector index
// modulo the depth whatever the source. Two at every width: deeper rings
// measured 3-5% faster at 4096 rows for the 4- and 6-wide reads but 1-2%
// slower at 2048, and up to 10% slower for the 12-wide read. The kernels take
// the depth as a template argument; the 4-, 6- and 8-wide ones are also built
// with every vector of a source in flight (a depth equal to the width), which
// the host takes for launches of 6 to 7 rows per CU (4 to 7 at width 8), where
// two loads per wave leave the memory idle.
constexpr int wave_depth(int) { return 2; }

// One source row of the fold: its resource (empty for an invalid MoE pick or a
// missing residual, so its loads read 0) and, for MoE, its gate.
struct RowSource {
  Rsrc r;
  float g;
};

template <Source S>
__device__ __forceinline__ RowPicks row_picks(const RowArgs& a, int64_t row, int lane) {
  if constexpr (S == Source::Moe) return load_picks(a, row, a.nsrc, lane);
  return RowPicks{};
}

template <Source S>
__device__ __forceinline__ RowSource row_source(const RowArgs& a, const RowPicks& picks, int64_t row, int p) {
  const int rb = a.H * 2;
  if (p == a.nsrc) return {row_rsrc(a.res + row * a.ld_res, a.has_residual ? rb : 0), 1.0f};
  if constexpr (S == Source::Partials) {
    return {row_rsrc(a.src[p] + row * a.ld_src, rb), 1.0f};
  } else {
    // a dropped pick reads zeros through an empty resource with a zero gate: it adds nothing,
    // whatever its gate holds
    int64_t e;
    float g;
    resolve_pick(a, picks, p, e, g);
    return {row_rsrc(a.experts + (e < 0 ? 0 : e) * a.ld_e, e < 0 ? 0 : rb), g};
  }
}

// The first two sources of a row of owed partials (n >= 1, which the dispatchers check): source 0
// is partial 0; source 1 is partial 1, or for n = 1 the row after the partials (`kTail`: the
// residual of a fold or a snapshot, the extra row of add_to_output, nothing for complete_only),
// the same rows row_source and complete_source give. Every pointer is read before the choice,
// which is then a select: the kernel's argument loads issue together, where a branch per choice
// cost one dependent round trip each before the row's first loads (about 1% on the 2048-row
// folds, whose rows all start at once).
template <Tail kTail>
__device__ __forceinline__ void first_partials(const RowArgs& a, int64_t row, int n, RowSource& cur,
                                               RowSource& next) {
  __builtin_assume(n >= 1);
  const int rb = a.H * 2;
  const uint16_t* p0 = a.src[0] + row * a.ld_src;
  const uint16_t* p1 = a.src[1] + row * a.ld_src;
  const uint16_t* tail = kTail == Tail::Extra ? a.extra + row * a.ld_extra : a.res + row * a.ld_res;
  const int tail_bytes = kTail == Tail::Extra ? rb : kTail == Tail::Residual ? (a.has_residual ? rb : 0) : 0;
  cur = {row_rsrc(p0, rb), 1.0f};
  next = {row_rsrc(n > 1 ? p1 : tail, n > 1 ? rb : tail_bytes), 1.0f};
}

__device__ __forceinline__ void load_weight8(const Rsrc& wr, int vec, u32x4& lo, u32x4& hi) {
  // the weight is shared by all rows: default cache policy, it stays in L2
  lo = __builtin_amdgcn_raw_buffer_load_b128(wr, vec * 32, 0, 0);
  hi = __builtin_amdgcn_raw_buffer_load_b128(wr, vec * 32 + 16, 0, 0);
}

// The pipeline over one source row: step v consumes the ring slot of vector v
// and refills it with the load D = wave_depth(VPT) vectors ahead, which for
// the last D vectors is the next source's first D. VPT is a multiple of D, so
// the slot of every load is its vector index mod D, whatever the source.
// One source vector into the running sum: a MoE pick adds g * t (the first
// with a zero start), a partial adds t (the first is copied).
template <Source S, bool kFirst>
__device__ __forceinline__ void add_source(float g, const float (&t)[8], float (&x)[8]) {
  if constexpr (S == Source::Moe) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = fmaf(g, t[e], kFirst ? 0.0f : x[e]);
  } else if constexpr (kFirst) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = t[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += t[e];
  }
}

template <Source S, int VPT, bool kFirst, int D>
__device__ __forceinline__ void fold_source(const RowSource& cur, const RowSource& next, int lane, uint4 (&ring)[D],
                                            float (&x)[VPT][8]) {
  static_assert(VPT % D == 0, "ring slots follow the vector index");
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    float t[8];
    bf16x8_to_f32(ring[v % D], t);
    ring[v % D] = v + D < VPT ? load16(cur.r, (lane + (v + D) * kWave) * 16)
                              : load16(next.r, (lane + (v + D - VPT) * kWave) * 16);
    add_source<S, kFirst>(cur.g, t, x[v]);
    pin8(x[v]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <Source S, int VPT, bool FP8, int D = wave_depth(VPT)>
__global__ __launch_bounds__(kWave) void wave_read_kernel(const RowArgs a) {
  static_assert(S == Source::Partials || S == Source::Moe, "one-wave rows fold partials or MoE picks");
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = a.nsrc;
  const Rsrc wr = row_rsrc(a.w, a.H * 4);
  const Rsrc res = row_rsrc(a.res + row * a.ld_res, a.H * 2);
  const float offset = a.gemma ? 1.0f : 0.0f;

  uint4 ring[D];
  u32x4 wlo[D], whi[D];
  const RowPicks picks = row_picks<S>(a, row, lane);
  RowSource cur, next;
  if constexpr (S == Source::Partials) {
    first_partials<Tail::Residual>(a, row, n, cur, next);  // the residual follows the partials
  } else {
    cur = row_source<S>(a, picks, row, 0);
    next = row_source<S>(a, picks, row, 1);
  }
#pragma unroll
  for (int v = 0; v < D; ++v) ring[v] = load16(cur.r, (lane + v * kWave) * 16);
  // the weights of the residual pass's first vectors, held until then
#pragma unroll
  for (int v = 0; v < D; ++v) load_weight8(wr, lane + v * kWave, wlo[v], whi[v]);
  __builtin_amdgcn_sched_barrier(0);

  float x[VPT][8];
  fold_source<S, VPT, true>(cur, next, lane, ring, x);
  for (int p = 1; p < n; ++p) {
    cur = next;
    next = row_source<S>(a, picks, row, p + 1);  // p + 1 == n: the residual
    fold_source<S, VPT, false>(cur, next, lane, ring, x);
  }

  // The residual pass: each vector is finished here. The residual is stored at
  // once (lanes past the end of the row address beyond the row resource and
  // are dropped), x^2 and |x w| are accumulated and only x w is kept, so the
  // row never holds x and w together.
  float ss = 0.0f, mx = 0.0f;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    float t[8];
    bf16x8_to_f32(ring[v % D], t);
    const u32x4 lo = wlo[v % D], hi = whi[v % D];
    if (v + D < VPT) {
      ring[v % D] = load16(next.r, (lane + (v + D) * kWave) * 16);
      load_weight8(wr, lane + (v + D) * kWave, wlo[v % D], whi[v % D]);
    }
    const float w[8] = {__uint_as_float(lo.x) + offset, __uint_as_float(lo.y) + offset,
                        __uint_as_float(lo.z) + offset, __uint_as_float(lo.w) + offset,
                        __uint_as_float(hi.x) + offset, __uint_as_float(hi.y) + offset,
                        __uint_as_float(hi.z) + offset, __uint_as_float(hi.w) + offset};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[v][e] = t[e] + x[v][e];  // residual + contribution
    store16(res, (lane + v * kWave) * 16, f32_to_bf16x8(x[v]));
    ss += vector_ss(x[v]);  // this lane's vectors in index order: the shape-free order of row_reduce
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[v][e] = x[v][e] * w[e];
      mx = fmaxf(mx, fabsf(x[v][e]));
    }
    pin8(x[v]);
    __builtin_amdgcn_sched_barrier(0);
  }

  ss = wave_sum(ss);
  if constexpr (FP8) mx = wave_max(mx);
  const float inv = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  if constexpr (!FP8) {
    const Rsrc yr = row_rsrc(a.y + row * a.ld_y, a.H * 2);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[v][e] * inv;
      store16(yr, (lane + v * kWave) * 16, f32_to_bf16x8(y));
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // max_h |y_h| = (max_h |x_h w_h|) inv exactly (rounding is monotone)
    const float amax = mx * inv;
    const float scale = amax / 448.0f;
    const float rcp = scale > 0.0f ? 1.0f / scale : 0.0f;
    const Rsrc qr = row_rsrc(a.q + row * a.ld_q, a.H);
    const auto codes = [&](auto divide) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float y[8], t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[v][e] * inv;
        fp8_inputs<decltype(divide)::value>(y, scale, rcp, t);
        store8(qr, (lane + v * kWave) * 8, f32_to_e4m3x8(t));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (fp8_divide(rcp))  // uniform across the row
      codes(std::true_type{});
    else
      codes(std::false_type{});
    if (lane == 0) a.scale[row] = scale;
  }
}

// ---------------------------------------------------------------------------
// complete_only, add_to_output and snapshot with one wavefront per row: the
// pipeline of wave_read_kernel over the P partials or k picks, then the tail:
// nothing, the extra row (add_to_output) or the residual (snapshot); the last
// source's pass stores each finished vector at once. The sums run in
// complete_kernel's order, including the zero that stands for the residual
// when nothing is folded (0 + s turns a -0 sum into +0), so the output is
// bitwise the same under both kernels.
// ---------------------------------------------------------------------------

// Source p of a complete: p < n a partial or pick, p == n the tail row when
// there is one; any other p is an empty row (its loads read 0).
template <Source S, Tail kTail>
__device__ __forceinline__ RowSource complete_source(const RowArgs& a, const RowPicks& picks, int64_t row, int p) {
  if (p < a.nsrc || (kTail == Tail::Residual && p == a.nsrc)) return row_source<S>(a, picks, row, p);
  const bool extra = kTail == Tail::Extra && p == a.nsrc;
  return {row_rsrc(extra ? a.extra + row * a.ld_extra : a.res, extra ? a.H * 2 : 0), 1.0f};
}

// The last source's pass: add it and store every vector as soon as it is final.
template <Source S, int VPT, bool kFirst, Tail kTail, int D>
__device__ __forceinline__ void store_source(const RowSource& cur, int lane, uint4 (&ring)[D], float (&x)[VPT][8],
                                             const Rsrc& out) {
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    float t[8];
    bf16x8_to_f32(ring[v % D], t);
    if (v + D < VPT) ring[v % D] = load16(cur.r, (lane + (v + D) * kWave) * 16);
    if constexpr (kTail == Tail::Extra) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[v][e] = (0.0f + x[v][e]) + t[e];
    } else if constexpr (kTail == Tail::Residual) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[v][e] = t[e] + x[v][e];
    } else {
      add_source<S, kFirst>(cur.g, t, x[v]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[v][e] = 0.0f + x[v][e];
    }
    store16(out, (lane + v * kWave) * 16, f32_to_bf16x8(x[v]));
    pin8(x[v]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <Source S, int VPT, Tail kTail, int D = wave_depth(VPT)>
__global__ __launch_bounds__(kWave) void wave_complete_kernel(const RowArgs a) {
  static_assert(S == Source::Partials || S == Source::Moe, "one-wave rows complete partials or MoE picks");
  static_assert(kTail != Tail::Residual || S == Source::Partials, "a snapshot folds partials");
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = a.nsrc;
  const int folded = kTail != Tail::None ? n : n - 1;  // sources before the stored one
  const Rsrc out = row_rsrc(a.y + row * a.ld_y, a.H * 2);
  const RowPicks picks = row_picks<S>(a, row, lane);

  uint4 ring[D];
  RowSource cur, next;
  if constexpr (S == Source::Partials) {
    first_partials<kTail>(a, row, n, cur, next);
  } else {
    cur = complete_source<S, kTail>(a, picks, row, 0);
    next = complete_source<S, kTail>(a, picks, row, 1);
  }
#pragma unroll
  for (int v = 0; v < D; ++v) ring[v] = load16(cur.r, (lane + v * kWave) * 16);
  __builtin_amdgcn_sched_barrier(0);

  float x[VPT][8];
  if (kTail == Tail::None && folded == 0) {  // one partial or pick and nothing after it
    store_source<S, VPT, true, Tail::None>(cur, lane, ring, x, out);
    return;
  }
  fold_source<S, VPT, true>(cur, next, lane, ring, x);
  for (int p = 1; p < folded; ++p) {
    cur = next;
    next = complete_source<S, kTail>(a, picks, row, p + 1);
    fold_source<S, VPT, false>(cur, next, lane, ring, x);
  }
  cur = next;
  store_source<S, VPT, false, kTail>(cur, lane, ring, x, out);
}

// ---------------------------------------------------------------------------
// Host-side dispatch tables
// ---------------------------------------------------------------------------
using KernelFn = void (*)(RowArgs);

template <Source S, int VPT, bool FP8, bool kNt = false, int... I>
constexpr std::array<KernelFn, sizeof...(I)> read_table(std::integer_sequence<int, I...>) {
  return {{&read_kernel<S, I + 1, VPT, FP8, kNt>...}};
}

template <Source S, int VPT, bool kFold, int... I>
constexpr std::array<KernelFn, sizeof...(I)> complete_table(std::integer_sequence<int, I...>) {
  return {{&complete_kernel<S, I + 1, VPT, kFold>...}};
}

inline hipError_t launch_kernel(KernelFn fn, const RowArgs& a, const Launch& l, hipStream_t stream) {
  RowArgs copy = a;
  void* args[] = {&copy};
  if (l.start || l.stop)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)l.rows), dim3((unsigned)l.threads),
                              args, 0, stream, l.start, l.stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)l.rows), dim3((unsigned)l.threads),
                         args, 0, stream);
}

inline int vpt_slot(int vpt) { return vpt == 1 ? 0 : vpt == 2 ? 1 : vpt == 4 ? 2 : -1; }

// Workgroups of a one-wavefront kernel that a compute unit holds at once (its
// occupancy, which its VGPR count sets), asked of the runtime once and kept in
// `cache` (0: not asked yet, -1: the runtime could not tell; returns 0 then).
inline int occupancy_rows(KernelFn fn, std::atomic<int>& cache) {
  int n = cache.load();
  if (n == 0) {
    int blocks = 0;
    n = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(fn), kWave, 0) ==
                    hipSuccess && blocks > 0
            ? blocks
            : -1;
    cache.store(n);
  }
  return n > 0 ? n : 0;
}

}  // namespace bnd
