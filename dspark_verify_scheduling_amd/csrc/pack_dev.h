// Device side of the compact ragged layout, shared by the pack kernel and
// the fused plan+pack kernel.
//
// Method sources:
//   "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §五 (compact mode
//     packs only the selected rows, e.g. A0 A1 | B0 | C0 C1 C2 C3) and §六
//     (cu_seqlens_q = [0,2,3,7] for verify_lens [2,1,4]).
//   "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit" (akiyangdev) §三
//     (verify ids = anchor followed by the drafts; the anchor plus the
//     selected draft prefix is front-packed).
//   "DSpark 接入 SGLang" (yingzheng), ragged verify, and "DSpark
//     confidence-scheduled speculative decoding" (charlestar), graph tiers:
//     the packed total is rounded up to the smallest captured tier.
#pragma once

#include "common.h"

namespace dspark {

// Inputs of the packed rows that thread `threadIdx.x` writes in its first
// NPRE passes over the B * (gamma + 1) verify slots (slot f = tid + q *
// NTHREADS): the token id (anchor or draft) and the request's prefix length.
// Loading them at kernel start hides their latency behind earlier work.
template <int NTHREADS, int NPRE>
struct PackPrefetch {
  int id[NPRE > 0 ? NPRE : 1];
  int prefix[NPRE > 0 ? NPRE : 1];
  __device__ void load(const PackArgs& a) {
    const int G = a.gamma, rows = a.B * (G + 1);
    const SmallDiv per_req(G + 1);  // rows < 2^15
#pragma unroll
    for (int q = 0; q < NPRE; ++q) {
      const int f = threadIdx.x + q * NTHREADS;
      id[q] = 0;
      prefix[q] = 0;
      if (f < rows) {
        const int r = per_req.quo(f);
        const int j = f - r * (G + 1);
        id[q] = j ? a.drafts[(size_t)r * G + (j - 1)] : a.anchors[r];
        prefix[q] = a.prefix ? a.prefix[r] : 0;
      }
    }
  }
};

// The tier table one entry per lane (lane l < ntiers holds tiers[l]), loaded
// at kernel start so that picking the tier needs no load.
__device__ inline int load_tier_lane(const PackArgs& a) {
  const int l = lane_id();
  return a.tiers[l < a.ntiers ? l : 0];
}

// The first tier >= total, else the last tier (tiers ascend), from the
// per-lane table; wave-uniform, called by every lane of the wave.
__device__ inline int pick_tier(int tier_lane, int ntiers, int total) {
  const int l = lane_id();
  const unsigned long long m = __ballot(l < ntiers && tier_lane >= total);
  const int i = m ? (int)__builtin_ctzll(m) : ntiers - 1;
  return __builtin_amdgcn_readlane(tier_lane, i);
}

// Packs B requests whose (already clamped) lengths sit in LDS `lens`,
// writing cu_seqlens into LDS `cu` (B + 1 entries) and to global memory.
// Block-wide: every thread of the NTHREADS-thread workgroup must call it.
// `status` is OR-ed into meta[2] by thread 0 at the end. `tier_lane` is
// load_tier_lane's value; `pre` holds the inputs of this thread's first NPRE
// slots (see PackPrefetch).
template <int NTHREADS, int NPRE = 0>
__device__ void pack_block(const PackArgs& a, const int32_t* lens, int32_t* cu, int* wsum,
                           int tier_lane, int status,
                           const PackPrefetch<NTHREADS, NPRE>* pre = nullptr) {
  const int tid = threadIdx.x;
  const int B = a.B, G = a.gamma;
  const int ipt = (B + NTHREADS - 1) / NTHREADS;
  const int r0 = tid * ipt;
  int local = 0;
  for (int t = 0; t < ipt; ++t) {
    if (r0 + t < B) local += lens[r0 + t];
  }
  int total;
  // wsum is not written again: no closing barrier
  int run = block_excl_scan_open<int, NTHREADS>(local, wsum, &total);
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
  }
  const int tier = pick_tier(tier_lane, a.ntiers, total);
  __syncthreads();
  const int rows = B * (G + 1);  // < 2^15
  const SmallDiv per_req(G + 1);
#pragma unroll
  for (int q = 0; q < NPRE; ++q) {
    const int f = tid + q * NTHREADS;
    if (f < rows) {
      const int r = per_req.quo(f);
      const int j = f - r * (G + 1);
      if (j < lens[r]) {
        const int i = cu[r] + j;
        a.ids[i] = pre->id[q];
        if (a.req) a.req[i] = r;
        if (a.pos) a.pos[i] = pre->prefix[q] + j;
      }
    }
  }
  for (int f = tid + NPRE * NTHREADS; f < rows; f += NTHREADS) {
    const int r = per_req.quo(f);
    const int j = f - r * (G + 1);
    if (j < lens[r]) {
      const int i = cu[r] + j;
      a.ids[i] = j ? a.drafts[(size_t)r * G + (j - 1)] : a.anchors[r];
      if (a.req) a.req[i] = r;
      if (a.pos) a.pos[i] = (a.prefix ? a.prefix[r] : 0) + j;
    }
  }
  for (int i = total + tid; i < tier; i += NTHREADS) {
    a.ids[i] = 0;
    if (a.req) a.req[i] = -1;
    if (a.pos) a.pos[i] = 0;
  }
  if (tid == 0) {
    a.meta[0] = total;
    a.meta[1] = tier;
    a.meta[2] = status;
  }
}

}  // namespace dspark
