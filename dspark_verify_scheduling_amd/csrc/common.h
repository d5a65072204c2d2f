// Internal declarations shared by the HIP kernels of libdspark (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;

// ---------------------------------------------------------------- kernels

struct PlanArgs {
  int B, gamma, kind, lmin, lmax, b_lo, b_hi, n_sort;
  float eps, bias;
  const float* conf;
  const float* temps;
  const float* alpha;
  const float* theta;
  int32_t* lens;
  int32_t* meta;
  double* val;
  float* surv_out;
  double* sweep;
};
constexpr int kPlanThreads = 1024;
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
size_t plan_lds_bytes(int B, int n_sort);

struct PackArgs {
  int B, gamma, ntiers;
  const int32_t* lens;
  const int32_t* anchors;
  const int32_t* drafts;
  const int32_t* prefix;
  int32_t* cu;
  int32_t* ids;
  int32_t* req;
  int32_t* pos;
  int32_t* meta;
  int32_t tiers[DSPARK_MAX_TIERS];
};
constexpr int kPackThreads = 1024;
hipError_t launch_pack(const PackArgs& a, hipStream_t s);

struct AcceptArgs {
  const unsigned char* logits;
  int64_t ld_bytes;
  int V, max_rows, B, gamma;
  int chunks;      // units per row
  int chunk_vecs;  // 16-byte vectors per unit
  int nvec;        // whole 16-byte vectors per row
  int tail;        // elements after the last whole vector
  const int32_t* cu;
  const int32_t* drafts;
  const int32_t* prefix;
  int32_t* row_am;
  int32_t* num_correct;
  int32_t* bonus;
  int32_t* commit;
  int32_t* out_tokens;
  int32_t* new_seq;
  uint8_t* mask;
  int32_t* meta;
  unsigned long long* partials;  // [max_rows * chunks] (key, index) per unit
};
constexpr int kAccThreads = 256;
constexpr int kAccVecsPerThread = 8;
constexpr int kAccMaxChunkVecs = kAccThreads * kAccVecsPerThread;
hipError_t launch_accept(const AcceptArgs& a, dspark_dtype dt, int grid, hipStream_t s);

struct TvArgs {
  const unsigned char* q;
  int64_t ldq_bytes;
  const unsigned char* p;
  int64_t ldp_bytes;
  int V, B, gamma, rows_per_req;
  int nvec, tail;
  float* a_out;
  float* s_out;
};
constexpr int kTvThreads = 256;
hipError_t launch_tv(const TvArgs& a, dspark_dtype dt, hipStream_t s);

// ---------------------------------------------------------------- helpers

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ inline T wave_sum(T v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <typename T>
__device__ inline T wave_incl_scan(T v) {
  const int lane = lane_id();
  for (int d = 1; d < kWave; d <<= 1) {
    T n = __shfl_up(v, d, kWave);
    if (lane >= d) v += n;
  }
  return v;
}

// Exclusive scan over the block. `wsum` needs (waves + 1) slots. Returns the
// exclusive prefix of this thread's value; *total receives the block total.
template <typename T, int NTHREADS>
__device__ inline T block_excl_scan(T v, T* wsum, T* total) {
  constexpr int kWaves = NTHREADS / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  T incl = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    T w = lane < kWaves ? wsum[lane] : T(0);
    T wi = wave_incl_scan(w);
    if (lane < kWaves) wsum[lane] = wi - w;  // exclusive wave offsets
    if (lane == kWaves - 1) wsum[kWaves] = wi;
  }
  __syncthreads();
  T res = wsum[wave] + incl - v;
  *total = wsum[kWaves];
  __syncthreads();
  return res;
}

template <typename T, int NTHREADS>
__device__ inline T block_sum(T v, T* wsum) {
  constexpr int kWaves = NTHREADS / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  T t = T(0);
  for (int i = 0; i < kWaves; ++i) t += wsum[i];
  __syncthreads();
  return t;
}

}  // namespace dspark
