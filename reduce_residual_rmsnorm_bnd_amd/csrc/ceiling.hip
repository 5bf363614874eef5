// ceiling.hip -- measurement support, not part of the boundary path.
//
// A kernel with a boundary call's memory access mix and none of its arithmetic: for every
// 16-byte vector of a row it reads n rows and writes one or two (the second may be one byte per
// element, as the fp8 read's codes beside its bf16 residual), one row per workgroup, through
// the same per-row buffer resources and cache policy (non-temporal loads, sc1 stores) as the
// boundary kernels. The prefill fold's mix is nine reads (eight partials and the residual) and two
// writes (the residual and the normalised output); complete_only's is eight and one, a snapshot's
// or add_to_output's nine and one. The loaded vectors are combined with XOR so that every load is
// consumed and every store depends on all of them. With eight vectors per thread the stream
// follows the one-wavefront boundary kernels' order (ring_stream below); with one, two or four a
// thread issues a source's loads together. Its rate on a device is what that memory system
// delivers for the stream in this layout; each call is compared with its own mix as context.
// A gathering variant reads eight of
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
  int out1_bytes;  // out1's bytes per element: 2, or 1 (as the fp8 read's codes: 8 bytes per vector)
};

// Eight vectors per thread stream as the one-wavefront boundary kernels do: source after source,
// each thread's vectors of a source in order, two loads in flight through a ring that runs on
// across source boundaries (the next source's first vectors load while this one's last vectors
// are consumed), and during the last source's pass each finished vector stored at once to the
// first output, as those kernels store the residual (or a complete's output); a second output
// is stored after the stream, as they store y. `source_of(p)` is the resource of source p.
template <int VPT, bool kStore>
__device__ __forceinline__ void ring_pass(const bnd::Rsrc& cur, const bnd::Rsrc& next, const bnd::Rsrc& out,
                                          const int (&off)[VPT], uint4 (&ring)[2], uint4 (&acc)[VPT]) {
  static_assert(VPT % 2 == 0, "a ring slot is the vector index mod 2");
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const uint4 t = ring[v & 1];
    ring[v & 1] = v + 2 < VPT ? bnd::load16(cur, off[v + 2]) : bnd::load16(next, off[v + 2 - VPT]);
    acc[v].x ^= t.x; acc[v].y ^= t.y; acc[v].z ^= t.z; acc[v].w ^= t.w;
    asm volatile("" : "+v"(acc[v].x), "+v"(acc[v].y), "+v"(acc[v].z), "+v"(acc[v].w));
    if constexpr (kStore) bnd::store16(out, off[v], acc[v]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// kN > 0: a source count known at compile time, the loop unrolled (the gathering stream, whose
// eight row indices then load together before the first pass, as the MoE finalize fetches its
// picks once per row); kN = 0: n_src (>= 1) at run time.
template <int VPT, int kN, typename SourceOf>
__device__ __forceinline__ void ring_stream(int n_src, SourceOf source_of, const bnd::Rsrc& out,
                                            const int (&off)[VPT], uint4 (&acc)[VPT]) {
  // After the last source the refills read an empty resource (zeros, no memory access), so every
  // step issues its load. The first source's pass runs before the loop, as in the boundary
  // kernels: both edges into the loop then leave the same loads outstanding in the same order,
  // and the compiler waits for one load at a time instead of draining the ring at each source.
  const bnd::Rsrc empty = bnd::row_rsrc(nullptr, 0);
  if constexpr (kN > 0) n_src = kN;
  uint4 ring[2];
  bnd::Rsrc cur = source_of(0);
  ring[0] = bnd::load16(cur, off[0]);
  ring[1] = bnd::load16(cur, off[1]);
  if (n_src == 1) {
    ring_pass<VPT, true>(cur, empty, out, off, ring, acc);
    return;
  }
  bnd::Rsrc next = source_of(1);
  ring_pass<VPT, false>(cur, next, out, off, ring, acc);
  if constexpr (kN > 0) {
#pragma unroll
    for (int p = 1; p < kN - 1; ++p) {
      cur = next;
      next = source_of(p + 1);
      ring_pass<VPT, false>(cur, next, out, off, ring, acc);
    }
  } else {
    for (int p = 1; p < n_src - 1; ++p) {
      cur = next;
      next = source_of(p + 1);
      ring_pass<VPT, false>(cur, next, out, off, ring, acc);
    }
  }
  ring_pass<VPT, true>(next, empty, out, off, ring, acc);  // the last source
}

template <int VPT>
__global__ __launch_bounds__(bnd::kMaxThreads) void mix_kernel(const MixArgs a) {
  const int64_t row = blockIdx.x;
  const int nthr = blockDim.x;
  int off[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) off[v] = (threadIdx.x + v * nthr) * 16;
  uint4 acc[VPT];
  const bnd::Rsrc o0 = bnd::row_rsrc(a.out0 + row * a.ld, a.row_bytes);
  if constexpr (VPT == 8) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) acc[v] = make_uint4(0u, 0u, 0u, 0u);
    ring_stream<VPT, 0>(a.n_src, [&](int p) { return bnd::row_rsrc(a.src[p] + row * a.ld, a.row_bytes); }, o0,
                        off, acc);
  } else {
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
  }
  if constexpr (VPT != 8) {  // the ring stored the first output during its last pass
#pragma unroll
    for (int v = 0; v < VPT; ++v) bnd::store16(o0, off[v], acc[v]);
  }
  if (a.out1 && a.out1_bytes == 1) {
    // one byte per element: the first 8 bytes of each 16-byte vector, at half its offset
    const bnd::Rsrc o1 = bnd::row_rsrc(reinterpret_cast<uint8_t*>(a.out1) + row * a.ld, a.row_bytes / 2);
#pragma unroll
    for (int v = 0; v < VPT; ++v) bnd::store8(o1, off[v] / 2, make_uint2(acc[v].x, acc[v].y));
  } else if (a.out1) {
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
  // source p < 8: row idx[row * 8 + p] of rows_src (an index outside the rows reads zeros);
  // source 8: row `row` of src8
  const auto source_of = [&](int p) {
    if (p < kSources - 1) {
      const int64_t e = a.idx[row * (kSources - 1) + p];
      const bool valid = e >= 0 && e < a.n_src_rows;
      return bnd::row_rsrc(a.rows_src + (valid ? e : 0) * a.ld, valid ? a.row_bytes : 0);
    }
    return bnd::row_rsrc(a.src8 + row * a.ld, a.row_bytes);
  };
  const bnd::Rsrc o0 = bnd::row_rsrc(a.out0 + row * a.ld, a.row_bytes);
  const bnd::Rsrc o1 = bnd::row_rsrc(a.out1 + row * a.ld, a.row_bytes);
  if constexpr (VPT == 8) {
    ring_stream<VPT, kSources>(kSources, source_of, o0, off, acc);
  } else {
#pragma unroll
    for (int p = 0; p < kSources; ++p) {
      const bnd::Rsrc r = source_of(p);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const uint4 t = bnd::load16(r, off[v]);
        acc[v].x ^= t.x; acc[v].y ^= t.y; acc[v].z ^= t.z; acc[v].w ^= t.w;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    if constexpr (VPT != 8) bnd::store16(o0, off[v], acc[v]);  // VPT 8: stored during the last pass
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
static int launch_mix(const void* const* src, int n_src, void* out0, void* out1, int out1_bytes, int64_t rows,
                      int64_t ld, int64_t row_elems, int threads, int vpt, hipStream_t stream) {
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
  if (!aligned16(out0) || (out1 && (reinterpret_cast<uintptr_t>(out1) & (out1_bytes == 1 ? 7 : 15)))) return -1;
  a.out0 = static_cast<uint16_t*>(out0);
  a.out1 = static_cast<uint16_t*>(out1);
  a.ld = ld;
  a.row_bytes = (int)(row_elems * 2);
  a.n_src = n_src;
  a.out1_bytes = out1_bytes;
  void* args[] = {&a};
  const void* fn = vpt == 1   ? reinterpret_cast<const void*>(&mix_kernel<1>)
                   : vpt == 2 ? reinterpret_cast<const void*>(&mix_kernel<2>)
                   : vpt == 4 ? reinterpret_cast<const void*>(&mix_kernel<4>)
                              : reinterpret_cast<const void*>(&mix_kernel<8>);
  return (int)hipLaunchKernel(fn, dim3((unsigned)rows), dim3((unsigned)threads), args, 0, stream);
}

extern "C" __attribute__((visibility("default"))) int bnd_ceiling_mix(
    const void* const* src, int n_src, void* out0, void* out1, int64_t rows, int64_t ld, int64_t row_elems,
    int threads, int vpt, hipStream_t stream) {
  return launch_mix(src, n_src, out0, out1, 2, rows, ld, row_elems, threads, vpt, stream);
}

// As bnd_ceiling_mix with a second output of one byte per element, as the fp8 read writes its
// codes beside the bf16 residual: out1 (8-byte aligned, required) is [rows, ld] bytes, and each
// 16-byte vector of a row stores its first 8 bytes there at half its offset.
extern "C" __attribute__((visibility("default"))) int bnd_ceiling_mix_byte_out1(
    const void* const* src, int n_src, void* out0, void* out1, int64_t rows, int64_t ld, int64_t row_elems,
    int threads, int vpt, hipStream_t stream) {
  if (!out1) return -1;
  return launch_mix(src, n_src, out0, out1, 1, rows, ld, row_elems, threads, vpt, stream);
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
