// Pack kernel: verify_lens -> cu_seqlens, front-packed verify rows, tier.
//
// Method sources:
//   "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §五 (compact mode
//     packs only the selected rows, e.g. A0 A1 | B0 | C0 C1 C2 C3) and §六
//     (cu_seqlens_q = [0,2,3,7] for verify_lens [2,1,4]).
//   "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit" (akiyangdev) §三
//     (verify ids = anchor followed by the drafts; BuildRaggedVerifyWindow
//     front-packs the anchor plus the selected draft prefix).
//   "DSpark 接入 SGLang" (yingzheng), ragged verify, and "DSpark
//     confidence-scheduled speculative decoding" (charlestar), graph tiers:
//     the packed total is rounded up to the smallest captured tier.
//
// One workgroup of 1024 threads (B <= 8192): each thread owns up to eight
// consecutive requests for the block scan. The flat (request, row) space is
// then walked with a block-stride loop so that consecutive threads write
// consecutive packed rows.
#include "common.h"

namespace dspark {

namespace {

constexpr int kWaves = kPackThreads / kWave;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackArgs a) {
  extern __shared__ int32_t sh[];  // lens[B], cu[B + 1]
  __shared__ int w32[kWaves + 1];
  __shared__ int s_flags;
  __shared__ int s_tier;

  const int tid = threadIdx.x;
  const int B = a.B, G = a.gamma;
  int32_t* lens = sh;
  int32_t* cu = sh + B;
  if (tid == 0) s_flags = 0;
  __syncthreads();

  const int ipt = (B + kPackThreads - 1) / kPackThreads;
  const int r0 = tid * ipt;
  int local = 0, bad = 0;
  for (int t = 0; t < ipt; ++t) {
    const int r = r0 + t;
    if (r < B) {
      int l = a.lens[r];
      if (l < 1 || l > G + 1) {
        bad = 1;
        l = min(max(l, 1), G + 1);
      }
      lens[r] = l;
      local += l;
    }
  }
  if (bad) atomicOr(&s_flags, DSPARK_DATA_BAD_LENS);
  int total;
  int run = block_excl_scan<int, kPackThreads>(local, w32, &total);
  for (int t = 0; t < ipt; ++t) {
    const int r = r0 + t;
    if (r < B) {
      cu[r] = run;
      a.cu[r] = run;
      run += lens[r];
    }
  }
  if (tid == 0) {
    cu[B] = total;
    a.cu[B] = total;
    int tier = a.tiers[a.ntiers - 1];
    for (int i = 0; i < a.ntiers; ++i) {
      if (a.tiers[i] >= total) {
        tier = a.tiers[i];
        break;
      }
    }
    s_tier = tier;
  }
  __syncthreads();

  const int rows = B * (G + 1);
  for (int f = tid; f < rows; f += kPackThreads) {
    const int r = f / (G + 1);
    const int j = f - r * (G + 1);
    if (j < lens[r]) {
      const int i = cu[r] + j;
      a.ids[i] = j ? a.drafts[(size_t)r * G + (j - 1)] : a.anchors[r];
      if (a.req) a.req[i] = r;
      if (a.pos) a.pos[i] = (a.prefix ? a.prefix[r] : 0) + j;
    }
  }
  const int tier = s_tier;
  for (int i = total + tid; i < tier; i += kPackThreads) {
    a.ids[i] = 0;
    if (a.req) a.req[i] = -1;
    if (a.pos) a.pos[i] = 0;
  }
  if (tid == 0) {
    a.meta[0] = total;
    a.meta[1] = tier;
    a.meta[2] = s_flags;
  }
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(2 * a.B + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kPackThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace dspark
