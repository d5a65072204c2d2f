// Scatter of front-packed verify rows back to the strided [B, stride] layout.
//
// Method source: "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit"
// (akiyangdev) §三: after the target forward on the compact rows,
// ScatterCompactToStrided restores logits and hidden states to the uniform
// [bs x stride] logical layout so that accept can address them by fixed
// position; the rows a request did not verify are not recomputed, and
// verify_lens still says which results are valid.
//
// A pure copy, bound by HBM bandwidth: every valid packed row is read once
// (nontemporal, its last use) and written once to row r * stride + j. One
// 256-thread workgroup per (request, unit of up to 512 16-byte vectors)
// copies that unit of the request's rows, up to kScatterRows rows at a
// time with every load of the batch issued before its first store, so a
// request of many rows costs about one memory round trip per batch and there
// are no idle workgroups. A malformed request's workgroups exit at once.
// Workgroup 0 also validates every request and writes the status, so no
// other workgroup touches the meta words.
#include "common.h"

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bool request_ok(const ScatterArgs& a, int r, int total_eff, int* c0, int* len) {
  const int s = a.cu[r], e = a.cu[r + 1];
  *c0 = s;
  *len = e - s;
  return s >= 0 && e - s >= 1 && e - s <= a.stride && e <= total_eff;
}

__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(ScatterArgs a) {
  const int tid = threadIdx.x;
  const int total = a.cu[a.B];
  const int total_eff = min(max(total, 0), a.max_rows);
  if (blockIdx.x == 0) {
    int bad = total != total_eff;
    for (int r = tid; r < a.B; r += kScatterThreads) {
      int c0, len;
      bad |= !request_ok(a, r, total_eff, &c0, &len);
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) {
      a.meta[0] = total;
      a.meta[1] = bad ? DSPARK_DATA_BAD_LENS : 0;
    }
  }
  const int u = blockIdx.x;
  const int r = u / a.chunks;
  const int chunk = u - r * a.chunks;
  if (r >= a.B) return;  // the single workgroup of an empty batch
  int c0, len;
  if (!request_ok(a, r, total_eff, &c0, &len)) return;
  const int v0 = chunk * a.chunk_vecs;
  const int v1 = min(v0 + a.chunk_vecs, a.nvec);
  constexpr int kV = kScatterVecsPerThread, kR = kScatterRows;
  for (int j0 = 0; j0 < len; j0 += kR) {
    u32x4 x[kR][kV];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const u32x4* s0 = reinterpret_cast<const u32x4*>(a.src + (size_t)(c0 + j0 + i) * a.src_ld);
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        const int v = v0 + k * kScatterThreads + tid;
        x[i][k] = (u32x4){0u, 0u, 0u, 0u};  // a defined value: no wait before the load
        if (j0 + i < len && v < v1) x[i][k] = __builtin_nontemporal_load(s0 + v);
      }
    }
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      u32x4* d0 = reinterpret_cast<u32x4*>(a.dst + ((size_t)r * a.stride + j0 + i) * a.dst_ld);
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        const int v = v0 + k * kScatterThreads + tid;
        if (j0 + i < len && v < v1) d0[v] = x[i][k];
      }
    }
  }
  // bytes after the last whole vector
  if (chunk == a.chunks - 1 && tid < a.tail) {
    const size_t b = (size_t)a.nvec * 16 + tid;
    for (int j = 0; j < len; ++j) {
      a.dst[((size_t)r * a.stride + j) * a.dst_ld + b] = a.src[(size_t)(c0 + j) * a.src_ld + b];
    }
  }
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.chunks;
  hipLaunchKernelGGL(scatter_kernel, dim3(grid > 0 ? (unsigned)grid : 1u), dim3(kScatterThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace dspark
