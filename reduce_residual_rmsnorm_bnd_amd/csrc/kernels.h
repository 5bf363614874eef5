// kernels.h -- gfx950 kernels of the boundary path (included by the k_*.hip
// translation units, which instantiate them per source kind).
//
// One workgroup per token row. The row is split into 16-byte vectors of 8
// elements; thread t of a workgroup of `threads` lanes owns vectors
// t, t + threads, ... (VPT of them), so each load instruction of a wavefront
// reads 1 KiB of contiguous row. The row's work:
//   1. complete: issue the loads of all sources (P partials, or the k
//      gathered expert rows) and of the residual before any arithmetic, then
//      sum in fp32 in source order (the deferred all-reduce of the study
//      note's fusion point, on one GPU a sum over resident buffers);
//   2. fold: x = r + s in fp32 (guide, "Residual update and input read": the
//      plain update is an add and the read keeps the fp32 sum);
//   3. read: sum of squares over the row with a wave64 DPP reduction and one
//      LDS step across wavefronts, inv = 1/sqrt(ss/H + eps) (correctly
//      rounded divide and square root), y = x * inv * w;
//   4. store the residual as bf16 (round to nearest even, v_cvt_pk_bf16_f32)
//      and y as bf16, or as OCP e4m3 codes (v_cvt_pk_fp8_f32) with a
//      per-row fp32 scale.
// No atomics: the result is bitwise reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <utility>

#include "launch.h"

namespace bnd {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void store16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

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

// Row totals across the workgroup's wavefronts: one LDS slot per wave and a
// single barrier; every thread then adds the slots in wave order, so all
// threads hold the same, order-fixed result.
template <bool kWithMax>
__device__ __forceinline__ void block_reduce(float& ss, float& mx, float* lds_sum, float* lds_max) {
  ss = wave_sum(ss);
  if constexpr (kWithMax) mx = wave_max(mx);
  const int nw = blockDim.x / kWave;
  if (nw == 1) return;
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    lds_sum[wid] = ss;
    if constexpr (kWithMax) lds_max[wid] = mx;
  }
  __syncthreads();
  float t = 0.0f, m = 0.0f;
  for (int i = 0; i < nw; ++i) {
    t += lds_sum[i];
    if constexpr (kWithMax) m = fmaxf(m, lds_max[i]);
  }
  ss = t;
  mx = m;
}

// ---------------------------------------------------------------------------
// Loading and completing the contribution of one row: x[v][e] for the
// thread's VPT vectors. Lanes past the end of the row hold zeros.
// ---------------------------------------------------------------------------
// kFold = false computes the contribution s alone (complete_only).
template <Source S, int N, int VPT, bool kFold = true>
__device__ __forceinline__ void load_and_fold(const RowArgs& a, int64_t row, int tid, int nthr,
                                              const bool (&ok)[VPT], float (&x)[VPT][8]) {
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (S == Source::Partials) {
    uint4 c[N][VPT];
    uint4 r[VPT];
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const uint16_t* base = a.src[p] + row * a.ld_src;
#pragma unroll
      for (int v = 0; v < VPT; ++v) c[p][v] = ok[v] ? load16(base + (int64_t)(tid + v * nthr) * 8) : zero;
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v)
      r[v] = (kFold && ok[v] && a.has_residual) ? load16(a.res + row * a.ld_res + (int64_t)(tid + v * nthr) * 8)
                                       : zero;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float s[8], t[8], rv[8];
      bf16x8_to_f32(c[0][v], s);
#pragma unroll
      for (int p = 1; p < N; ++p) {
        bf16x8_to_f32(c[p][v], t);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += t[e];
      }
      bf16x8_to_f32(r[v], rv);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[v][e] = rv[e] + s[e];
    }
  } else if constexpr (S == Source::Moe) {
    int64_t er[N];
    float g[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int64_t e = a.idx[row * N + j];
      const bool valid = e >= 0 && e < a.n_expert_rows;
      er[j] = valid ? e : -1;
      g[j] = a.gate[row * N + j];
    }
    uint4 c[N][VPT];
    uint4 r[VPT];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint16_t* base = a.experts + (er[j] < 0 ? 0 : er[j]) * a.ld_e;
#pragma unroll
      for (int v = 0; v < VPT; ++v)
        c[j][v] = (ok[v] && er[j] >= 0) ? load16(base + (int64_t)(tid + v * nthr) * 8) : zero;
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v)
      r[v] = (kFold && ok[v] && a.has_residual) ? load16(a.res + row * a.ld_res + (int64_t)(tid + v * nthr) * 8)
                                       : zero;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float s[8], t[8], rv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        bf16x8_to_f32(c[j][v], t);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = fmaf(g[j], t[e], s[e]);
      }
      bf16x8_to_f32(r[v], rv);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[v][e] = rv[e] + s[e];
    }
  } else {
    // Input: the stack input x_in (enter); Residual: the stored residual (written read)
    const uint16_t* base = (S == Source::Input) ? a.x_in + row * a.ld_x : a.res + row * a.ld_res;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const uint4 raw = ok[v] ? load16(base + (int64_t)(tid + v * nthr) * 8) : zero;
      if constexpr (S == Source::Input) {
        if (ok[v] && a.copy_input) store16(a.res + row * a.ld_res + (int64_t)(tid + v * nthr) * 8, raw);
      }
      bf16x8_to_f32(raw, x[v]);
    }
  }
}

template <int VPT>
__device__ __forceinline__ void load_weight(const RowArgs& a, int tid, int nthr, const bool (&ok)[VPT],
                                            float (&w)[VPT][8]) {
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (ok[v]) {
      const float4* p = reinterpret_cast<const float4*>(a.w + (int64_t)(tid + v * nthr) * 8);
      lo = p[0];
      hi = p[1];
    }
    w[v][0] = lo.x; w[v][1] = lo.y; w[v][2] = lo.z; w[v][3] = lo.w;
    w[v][4] = hi.x; w[v][5] = hi.y; w[v][6] = hi.z; w[v][7] = hi.w;
  }
}

// ---------------------------------------------------------------------------
// The boundary read kernel: complete, fold, RMSNorm, stores.
// ---------------------------------------------------------------------------
template <Source S, int N, int VPT, bool FP8>
__global__ __launch_bounds__(kMaxThreads) void read_kernel(const RowArgs a) {
  __shared__ float lds_sum[kMaxThreads / kWave];
  __shared__ float lds_max[kMaxThreads / kWave];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  bool ok[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) ok[v] = (tid + v * nthr) < a.nvec;

  float x[VPT][8];
  load_and_fold<S, N, VPT>(a, row, tid, nthr, ok, x);
  float w[VPT][8];
  load_weight<VPT>(a, tid, nthr, ok, w);

  float ss = 0.0f, mx = 0.0f;
#pragma unroll
  for (int v = 0; v < VPT; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[v][e], x[v][e], ss);
  if constexpr (FP8) {
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[v][e] * w[v][e]));
  }
  block_reduce<FP8>(ss, mx, lds_sum, lds_max);
  const float inv = 1.0f / sqrtf(ss / (float)a.H + a.eps);

  if constexpr (S == Source::Partials || S == Source::Moe) {
#pragma unroll
    for (int v = 0; v < VPT; ++v)
      if (ok[v]) store16(a.res + row * a.ld_res + (int64_t)(tid + v * nthr) * 8, f32_to_bf16x8(x[v]));
  }

  if constexpr (!FP8) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (x[v][e] * inv) * w[v][e];
      if (ok[v]) store16(a.y + row * a.ld_y + (int64_t)(tid + v * nthr) * 8, f32_to_bf16x8(y));
    }
  } else {
    // y_h = (x_h w_h) inv. Rounding is monotone, so max_h |y_h| is exactly
    // (max_h |x_h w_h|) inv: the scale is fp32(max|y| / 448) of these y.
    const float amax = mx * inv;
    const float scale = amax / 448.0f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = (x[v][e] * w[v][e]) * inv;
        const float u = scale > 0.0f ? y / scale : 0.0f;
        t[e] = fminf(fmaxf(u, -448.0f), 448.0f);
      }
      if (ok[v]) *reinterpret_cast<uint2*>(a.q + row * a.ld_q + (int64_t)(tid + v * nthr) * 8) = f32_to_e4m3x8(t);
    }
    if (tid == 0) a.scale[row] = scale;
  }
}

// complete_only: the contribution alone, stored as bf16.
template <Source S, int N, int VPT>
__global__ __launch_bounds__(kMaxThreads) void complete_kernel(const RowArgs a) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  bool ok[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) ok[v] = (tid + v * nthr) < a.nvec;
  float s[VPT][8];
  load_and_fold<S, N, VPT, false>(a, row, tid, nthr, ok, s);
#pragma unroll
  for (int v = 0; v < VPT; ++v)
    if (ok[v]) store16(a.y + row * a.ld_y + (int64_t)(tid + v * nthr) * 8, f32_to_bf16x8(s[v]));
}

// ---------------------------------------------------------------------------
// Host-side dispatch tables
// ---------------------------------------------------------------------------
using KernelFn = void (*)(RowArgs);

template <Source S, int VPT, bool FP8, int... I>
constexpr std::array<KernelFn, sizeof...(I)> read_table(std::integer_sequence<int, I...>) {
  return {{&read_kernel<S, I + 1, VPT, FP8>...}};
}

template <Source S, int VPT, int... I>
constexpr std::array<KernelFn, sizeof...(I)> complete_table(std::integer_sequence<int, I...>) {
  return {{&complete_kernel<S, I + 1, VPT>...}};
}

inline hipError_t launch_kernel(KernelFn fn, const RowArgs& a, const Launch& l, hipStream_t stream) {
  RowArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)l.rows), dim3((unsigned)l.threads),
                         args, 0, stream);
}

inline int vpt_slot(int vpt) { return vpt == 1 ? 0 : vpt == 2 ? 1 : vpt == 4 ? 2 : -1; }

}  // namespace bnd
