// ceiling.hip -- measurement support, not part of the boundary path.
//
// A kernel with a boundary call's memory access mix and none of its arithmetic: for every
// 16-byte vector of a row it reads n rows and writes one or two, one row per workgroup, through
// the same per-row buffer resources and cache policy (non-temporal loads, sc1 stores) as the
// boundary kernels. The prefill fold's mix is nine reads (eight partials and the residual) and two
// writes (the residual and the normalised output); complete_only's is eight and one, a snapshot's
// or add_to_output's nine and one. The loaded vectors are combined with XOR so that every load is
// consumed and every store depends on all of them. Its rate on a device is what that memory
// system delivers for the stream in this layout; each call is compared with its own mix as
// context. A gathering variant reads eight of
// the nine rows through an int32 row index, as the MoE finalize reads its picks. An empty kernel
// gives the cost of a launch with no work, the floor under the per-boundary time of small
// batches. Built into its own library (libboundary_ceiling.so); the boundary library does not
// contain it.
#include <string.h>

#include "kernels.h"

namespace {

constexpr int kSources = 9;         // the gathering stream: eight gathered rows and one more
constexpr int kMaxMixSources = 16;

struct MixArgs {
  const uint16_t* src[kMaxMixSources];
  uint16_t* out0;
  uint16_t* out1;  // NULL: one output
  int64_t ld;      // elements between rows, same for every operand
  int row_bytes;   // bytes of a row that are read and written
  int n_src;       // 1..16
};

template <int VPT>
__global__ __launch_bounds__(bnd::kMaxThreads) void mix_kernel(const MixArgs a) {
  const int64_t row = blockIdx.x;
  const int nthr = blockDim.x;
  int off[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) off[v] = (threadIdx.x + v * nthr) * 16;
  uint4 acc[VPT];
  {
    const bnd::Rsrc r = bnd::row_rsrc(a.src[0] + row * a.ld, a.row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) acc[v] = bnd::load16(r, off[v]);
  }
  for (int p = 1; p < a.n_src; ++p) {
    const bnd::Rsrc r = bnd::row_rsrc(a.src[p] + row * a.ld, a.row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const uint4 t = bnd::load16(r, off[v]);
      acc[v].x ^= t.x; acc[v].y ^= t.y; acc[v].z ^= t.z; acc[v].w ^= t.w;
    }
  }
  const bnd::Rsrc o0 = bnd::row_rsrc(a.out0 + row * a.ld, a.row_bytes);
#pragma unroll
  for (int v = 0; v < VPT; ++v) bnd::store16(o0, off[v], acc[v]);
  if (a.out1) {
    const bnd::Rsrc o1 = bnd::row_rsrc(a.out1 + row * a.ld, a.row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) bnd::store16(o1, off[v], acc[v]);
  }
}

// The same stream with sources 0..7 gathered: source j of row t is row idx[t * 8 + j] of
// `rows_src`; source 8 is row t of `src8`.
struct GatherArgs {
  const uint16_t* rows_src;
  const int32_t* idx;
  const uint16_t* src8;
  uint16_t* out0;
  uint16_t* out1;
  int64_t ld;
  int64_t n_src_rows;  // rows of rows_src; an index outside [0, n_src_rows) reads zeros
  int row_bytes;
};

template <int VPT>
__global__ __launch_bounds__(bnd::kMaxThreads) void gather_kernel(const GatherArgs a) {
  const int64_t row = blockIdx.x;
  const int nthr = blockDim.x;
  int off[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) off[v] = (threadIdx.x + v * nthr) * 16;
  uint4 acc[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) acc[v] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int p = 0; p < kSources; ++p) {
    const uint16_t* base;
    int bytes = a.row_bytes;
    if (p < kSources - 1) {
      const int64_t e = a.idx[row * (kSources - 1) + p];
      const bool valid = e >= 0 && e < a.n_src_rows;
      base = a.rows_src + (valid ? e : 0) * a.ld;
      bytes = valid ? a.row_bytes : 0;
    } else {
      base = a.src8 + row * a.ld;
    }
    const bnd::Rsrc r = bnd::row_rsrc(base, bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const uint4 t = bnd::load16(r, off[v]);
      acc[v].x ^= t.x; acc[v].y ^= t.y; acc[v].z ^= t.z; acc[v].w ^= t.w;
    }
    // With eight vectors per thread a row's 72 loads (288 VGPRs) cannot all be in flight within
    // the 128 VGPRs of a 1024-thread workgroup: one source's loads at a time, as in mix_kernel,
    // instead of a spill to scratch.
    if constexpr (VPT >= 8) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) asm volatile("" : "+v"(acc[v].x), "+v"(acc[v].y), "+v"(acc[v].z), "+v"(acc[v].w));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const bnd::Rsrc o0 = bnd::row_rsrc(a.out0 + row * a.ld, a.row_bytes);
  const bnd::Rsrc o1 = bnd::row_rsrc(a.out1 + row * a.ld, a.row_bytes);
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    bnd::store16(o0, off[v], acc[v]);
    bnd::store16(o1, off[v], acc[v]);
  }
}

__global__ __launch_bounds__(bnd::kMaxThreads) void empty_kernel() {}

// An empty kernel that takes the boundary kernels' argument block (RowArgs, by value) and reads
// one field of it, as every boundary kernel does before its first load: the launch cost with the
// boundary's kernel arguments and their first scalar load, and no work. The store never runs (the
// host passes H = 0 and a NULL y).
__global__ __launch_bounds__(bnd::kMaxThreads) void empty_args_kernel(const bnd::RowArgs a) {
  if (a.H != 0 && threadIdx.x == 0) a.y[0] = 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// Launches the streaming kernel once on `stream`:
//   src        n_src (1..16) device pointers to [rows, ld] bf16 row-major operands (read)
//   out0/out1  device pointers to [rows, ld] bf16 operands (written; may not alias src); out1
//              may be NULL for one output
//   rows       grid size, one workgroup per row, 1 .. 2^31-1
//   row_elems  bf16 elements per row that are streamed, a multiple of 8, row_elems <= ld
//   threads    workgroup size, a multiple of 64 in [64, 1024]; vpt in {1, 2, 4, 8};
//              threads * vpt * 8 must cover row_elems
// Returns 0 on success, -1 on an invalid argument (nothing launched), or the hipError_t of the
// launch.
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_mix(
    const void* const* src, int n_src, void* out0, void* out1, int64_t rows, int64_t ld, int64_t row_elems,
    int threads, int vpt, hipStream_t stream) {
  if (!src || n_src < 1 || n_src > kMaxMixSources || !out0 || rows < 1 || rows > 0x7fffffff || row_elems < 8 ||
      row_elems % 8 || ld < row_elems || ld % 8 || row_elems * 2 > 0x7fffffff)
    return -1;
  if (threads < 64 || threads > bnd::kMaxThreads || threads % 64 || (vpt != 1 && vpt != 2 && vpt != 4 && vpt != 8) ||
      (int64_t)threads * vpt * 8 < row_elems || rows * threads > 0xffffffffll)
    return -1;
  MixArgs a = {};
  for (int p = 0; p < n_src; ++p) {
    if (!src[p] || !aligned16(src[p])) return -1;
    a.src[p] = static_cast<const uint16_t*>(src[p]);
  }
  if (!aligned16(out0) || (out1 && !aligned16(out1))) return -1;
  a.out0 = static_cast<uint16_t*>(out0);
  a.out1 = static_cast<uint16_t*>(out1);
  a.ld = ld;
  a.row_bytes = (int)(row_elems * 2);
  a.n_src = n_src;
  void* args[] = {&a};
  const void* fn = vpt == 1   ? reinterpret_cast<const void*>(&mix_kernel<1>)
                   : vpt == 2 ? reinterpret_cast<const void*>(&mix_kernel<2>)
                   : vpt == 4 ? reinterpret_cast<const void*>(&mix_kernel<4>)
                              : reinterpret_cast<const void*>(&mix_kernel<8>);
  return (int)hipLaunchKernel(fn, dim3((unsigned)rows), dim3((unsigned)threads), args, 0, stream);
}

// The prefill fold's mix: nine sources, two outputs (out1 must not be NULL).
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_mix_9r2w(
    const void* const* src, void* out0, void* out1, int64_t rows, int64_t ld, int64_t row_elems, int threads,
    int vpt, hipStream_t stream) {
  if (!out1) return -1;
  return bnd_ceiling_mix(src, 9, out0, out1, rows, ld, row_elems, threads, vpt, stream);
}

// Launches the empty kernel once on `stream`: `workgroups` (1 .. 2^31-1) workgroups of `threads`
// (a multiple of 64 in [64, 1024]) that do nothing. Returns 0 on success, -1 on an invalid
// argument (nothing launched), or the hipError_t of the launch.
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_empty(int64_t workgroups, int threads,
                                                                        hipStream_t stream) {
  if (workgroups < 1 || workgroups > 0x7fffffff || threads < 64 || threads > bnd::kMaxThreads || threads % 64 ||
      workgroups * threads > 0xffffffffll)
    return -1;
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&empty_kernel), dim3((unsigned)workgroups),
                              dim3((unsigned)threads), nullptr, 0, stream);
}

// Launches empty_args_kernel once on `stream`: as bnd_ceiling_empty, with a zeroed RowArgs block
// (sizeof(bnd::RowArgs) bytes of kernel arguments).
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_empty_args(int64_t workgroups, int threads,
                                                                             hipStream_t stream) {
  if (workgroups < 1 || workgroups > 0x7fffffff || threads < 64 || threads > bnd::kMaxThreads || threads % 64 ||
      workgroups * threads > 0xffffffffll)
    return -1;
  bnd::RowArgs a;
  memset(&a, 0, sizeof a);
  void* args[] = {&a};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&empty_args_kernel), dim3((unsigned)workgroups),
                              dim3((unsigned)threads), args, 0, stream);
}

// The size in bytes of the boundary kernels' argument block.
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_args_bytes(void) { return (int)sizeof(bnd::RowArgs); }

// Launches the gathering 9:2 stream once on `stream`:
//   rows_src   device pointer to [n_src_rows, ld] bf16 rows, eight of which each output row reads
//   idx        device pointer to [rows * 8] int32 row indices into rows_src (gather form)
//   src8       device pointer to [rows, ld] bf16, the ninth source (row t for output row t)
//   out0/out1  device pointers to [rows, ld] bf16 outputs (written; may not alias the sources)
//   rows, row_elems, threads, vpt as for bnd_ceiling_mix_9r2w
// Returns 0 on success, -1 on an invalid argument (nothing launched), or the hipError_t of the
// launch.
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_gather_9r2w(
    const void* rows_src, int64_t n_src_rows, const int32_t* idx, const void* src8, void* out0, void* out1,
    int64_t rows, int64_t ld, int64_t row_elems, int threads, int vpt, hipStream_t stream) {
  if (!rows_src || !idx || !src8 || !out0 || !out1 || n_src_rows < 1 || rows < 1 || rows > 0x7fffffff ||
      row_elems < 8 || row_elems % 8 || ld < row_elems || ld % 8 || row_elems * 2 > 0x7fffffff)
    return -1;
  if (threads < 64 || threads > bnd::kMaxThreads || threads % 64 || (vpt != 1 && vpt != 2 && vpt != 4 && vpt != 8) ||
      (int64_t)threads * vpt * 8 < row_elems || rows * threads > 0xffffffffll)
    return -1;
  if (!aligned16(rows_src) || !aligned16(src8) || !aligned16(out0) || !aligned16(out1) ||
      (reinterpret_cast<uintptr_t>(idx) & 3))
    return -1;
  GatherArgs a;
  a.rows_src = static_cast<const uint16_t*>(rows_src);
  a.idx = idx;
  a.src8 = static_cast<const uint16_t*>(src8);
  a.out0 = static_cast<uint16_t*>(out0);
  a.out1 = static_cast<uint16_t*>(out1);
  a.ld = ld;
  a.n_src_rows = n_src_rows;
  a.row_bytes = (int)(row_elems * 2);
  void* args[] = {&a};
  const void* fn = vpt == 1   ? reinterpret_cast<const void*>(&gather_kernel<1>)
                   : vpt == 2 ? reinterpret_cast<const void*>(&gather_kernel<2>)
                   : vpt == 4 ? reinterpret_cast<const void*>(&gather_kernel<4>)
                              : reinterpret_cast<const void*>(&gather_kernel<8>);
  return (int)hipLaunchKernel(fn, dim3((unsigned)rows), dim3((unsigned)threads), args, 0, stream);
}
