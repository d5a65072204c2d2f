// Pack kernel: verify_lens -> cu_seqlens, front-packed verify rows, tier
// (see pack_dev.h for the method sources).
//
// One workgroup of 1024 threads (B <= 8192). Lengths outside [1, gamma + 1]
// set DSPARK_DATA_BAD_LENS and are clamped before packing.
#include "pack_dev.h"

namespace dspark {

namespace {

constexpr int kWaves = kPackThreads / kWave;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackArgs a) {
  extern __shared__ int32_t sh[];  // lens[B], cu[B + 1]
  __shared__ int w32[kWaves + 1];
  __shared__ int s_flags;
  const int tid = threadIdx.x;
  const int tier_lane = load_tier_lane(a);
  int32_t* lens = sh;
  int32_t* cu = sh + a.B;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  int bad = 0;
  for (int r = tid; r < a.B; r += kPackThreads) {
    int l = a.lens[r];
    if (l < 1 || l > a.gamma + 1) {
      bad = 1;
      l = min(max(l, 1), a.gamma + 1);
    }
    lens[r] = l;
  }
  if (bad) atomicOr(&s_flags, DSPARK_DATA_BAD_LENS);
  __syncthreads();
  pack_block<kPackThreads>(a, lens, cu, w32, tier_lane, s_flags);
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(2 * a.B + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kPackThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace dspark
