// Greedy accept: per-row argmax over the packed target logits, then the
// per-request leading-match count, bonus, commit and output tokens.
//
// Method sources:
//   "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit" (akiyangdev)
//     §四: verify row j's prediction checks draft j+1 (R checks A, A checks B);
//     §五: AcceptGreedy (target_predict = argmax, correct_len = leading
//          matches, bonus = prediction of the last valid input row),
//          FinalizeAcceptLens (commit = correct + 1, new_seq = prefix +
//          commit), BuildOutTokens (copy drafts, scatter bonus at correct).
//   "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §二: prefix_mask =
//     positions < num_correct_drafts; a match after the first mismatch is
//     not accepted.
//
// Two kernels on the caller's stream:
//
// 1. accept_argmax_kernel streams the total * V logits once. One
//    256-thread workgroup per (row, unit) of up to 2048 16-byte vectors
//    (32 KB); eight nontemporal 16-byte loads per thread are in flight before
//    any arithmetic. For bf16 the common case costs two packed 16-bit
//    instructions per pair of elements: a signed max of the raw bits (the
//    order of non-negative bf16 values) and an unsigned max that detects
//    negative NaNs. When the unit's maximum is positive and it holds no NaN,
//    only the lanes that hold the maximum search their registers for its
//    first position. Otherwise the unit is redone exactly from the same
//    registers with a total-order key (NaN highest, -0 == +0, lowest index
//    wins). Each unit writes one 64-bit (key, index) partial. The kernel has
//    no atomics and no cross-workgroup waits. The per-unit argmax lives in
//    argmax_unit.h, which the sampling accept's maximum pass shares.
// 2. accept_finalize_kernel: one wave per request merges its rows' partials,
//    counts the leading matches with a ballot, and writes the outputs; a
//    grid-stride pass writes the row argmax of every packed row.
//
// Cap-accept ("DSpark接入SGLang：用置信度驱动可变长度验证" (yingzheng), the
// three verify modes and the observability section; "DSpark 自适应 Verify
// 怎样分配候选预算" §五, cap-accept) runs the same two kernels on the fixed
// strided layout of B * (gamma + 1) rows: the leading matches are counted
// over all gamma drafts (the ceiling), then clipped to verify_len - 1, which
// commits what compact mode commits.
//
// The partials are fully rewritten by every call, so the workspace needs no
// initialization and holds no state between calls.
#include "argmax_unit.h"
#include "common.h"

namespace dspark {

namespace {

using namespace argmax;

constexpr int kMergeRound = 8;  // partial loads per row in flight at once

template <dspark_dtype DT>
__global__ __launch_bounds__(kAccThreads) void accept_argmax_kernel(AcceptArgs a) {
  __shared__ UnitSmem sm;
  const int tid = threadIdx.x;
  const int total = a.fixed_rows >= 0 ? a.fixed_rows : a.cu[a.B];
  const int total_eff = min(max(total, 0), a.max_rows);
  if (blockIdx.x == 0 && tid == 0) {
    a.meta[0] = total;
    a.meta[1] = total != total_eff ? DSPARK_DATA_BAD_LENS : 0;
  }
  const int u = blockIdx.x;
  if (u >= total_eff * a.chunks) return;
  const int row = u / a.chunks;
  const int chunk = u - row * a.chunks;
  const u32x4* rp = reinterpret_cast<const u32x4*>(a.logits + (size_t)row * a.ld_bytes);
  const int v0 = chunk * a.chunk_vecs;
  const int v1 = min(v0 + a.chunk_vecs, a.nvec);

  u32x4 d[kAccVecsPerThread];
#pragma unroll
  for (int j = 0; j < kAccVecsPerThread; ++j) {
    const int v = v0 + j * kAccThreads + tid;
    // -0.0 fill: below any positive value, never a NaN
    d[j] = (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    if (v < v1) d[j] = __builtin_nontemporal_load(rp + v);
  }

  const unsigned long long best =
      unit_best<DT>(d, v0, v1, a.logits + (size_t)row * a.ld_bytes, a.nvec, a.tail,
                    chunk == a.chunks - 1, sm);
  if (tid == 0) {
    a.partials[u] = best;
  }
}

// A partial's low word holds 0xFFFFFFFF - index, so the largest partial is
// the first position of the row's maximum.
__device__ inline int partial_index(unsigned long long m) {
  return (int)(0xFFFFFFFFu - (unsigned int)(m & 0xFFFFFFFFu));
}

__device__ inline int merge_row(const AcceptArgs& a, int row) {
  const unsigned long long* p = a.partials + (size_t)row * a.chunks;
  unsigned long long m = 0;
  for (int c = 0; c < a.chunks; ++c) m = p[c] > m ? p[c] : m;
  return partial_index(m);
}

// Maxima of two rows' partials (rows ra and rb, both below the number of rows
// the argmax pass wrote). Each round issues all sixteen loads before the
// first compare; chunk indices past the last repeat it, which leaves the
// maximum unchanged.
__device__ inline void merge_two_rows(const AcceptArgs& a, int ra, int rb, int& ia, int& ib) {
  const unsigned long long* pa = a.partials + (size_t)ra * a.chunks;
  const unsigned long long* pb = a.partials + (size_t)rb * a.chunks;
  const int last = a.chunks - 1;
  unsigned long long ma = 0, mb = 0;
  for (int c0 = 0; c0 <= last; c0 += kMergeRound) {
    unsigned long long va[kMergeRound], vb[kMergeRound];
#pragma unroll
    for (int k = 0; k < kMergeRound; ++k) {
      va[k] = pa[min(c0 + k, last)];
      vb[k] = pb[min(c0 + k, last)];
    }
#pragma unroll
    for (int k = 0; k < kMergeRound; ++k) {
      ma = va[k] > ma ? va[k] : ma;
      mb = vb[k] > mb ? vb[k] : mb;
    }
  }
  ia = partial_index(ma);
  ib = partial_index(mb);
}

// One wave per request (blockIdx.x = r), plus a grid-stride pass that writes
// the argmax of every row. CAP = false: packed rows cu[r] .. cu[r+1]-1.
// CAP = true: strided rows r * (gamma + 1) + j, every one of them computed.
// The loads come in two batches, each issued before anything waits on it:
// first the layout words, drafts and prefix; then every partial the wave
// needs (its row of the row pass and the request's rows). Stores follow.
template <bool CAP>
__global__ __launch_bounds__(kWave) void accept_finalize_kernel(AcceptArgs a) {
  __shared__ int am[DSPARK_MAX_GAMMA + 1];
  const int lane = threadIdx.x;
  const int G = a.gamma;
  const int r = blockIdx.x;
  const bool has_req = r < a.B;
  // first batch of loads: layout words, drafts, prefix
  const int total = CAP ? a.fixed_rows : a.cu[a.B];
  int c0 = 0, len = 0;  // first row, verify length
  if (has_req) {
    if constexpr (CAP) {
      c0 = r * (G + 1);
      len = a.lens[r];
    } else {
      c0 = a.cu[r];
      len = a.cu[r + 1] - c0;
    }
  }
  const int dr = (has_req && lane < G) ? a.drafts[(size_t)r * G + lane] : 0;
  const int prefix = (has_req && a.prefix) ? a.prefix[r] : 0;
  const int total_eff = min(max(total, 0), a.max_rows);
  bool ok;
  if constexpr (CAP) {
    ok = len >= 1 && len <= G + 1;
  } else {
    ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  }
  // second batch: the lane's row of the row pass and its row of the request,
  // read together at indices clamped into the rows written (results outside the
  // real ranges are discarded)
  const int i0 = blockIdx.x * kWave + lane;
  const int n_rows = CAP ? G + 1 : len;  // rows whose predictions are read
  const bool need = has_req && (CAP || ok);
  int g0 = 0, m0 = 0;
  if (total_eff > 0) {
    const int last = total_eff - 1;
    const int rr = min(min(max(c0, 0), last) + lane, last);
    merge_two_rows(a, min(i0, last), rr, g0, m0);
  }
  const int m1 = (need && lane + kWave < n_rows) ? merge_row(a, c0 + lane + kWave) : 0;
  if (i0 < total_eff) a.row_am[i0] = g0;
  for (int i = i0 + gridDim.x * kWave; i < total_eff; i += gridDim.x * kWave) {
    a.row_am[i] = merge_row(a, i);
  }
  if (!has_req) return;
  if (need) {
    if (lane < n_rows) am[lane] = m0;
    if (lane + kWave < n_rows) am[lane + kWave] = m1;
  }
  __syncthreads();
  int32_t* out = a.out_tokens + (size_t)r * (G + 1);
  // drafts compared: len - 1 of them, or all gamma for the ceiling
  const int n_chk = CAP ? G : len - 1;
  int c = 0;
  if (need) {
    // draft k (0-based, k < n_chk <= 64) against the prediction of row k
    const bool mismatch = lane < n_chk && dr != am[lane];
    const unsigned long long mm = __ballot(mismatch);
    c = mm ? (int)__builtin_ctzll(mm) : n_chk;
    if constexpr (CAP) {
      if (lane == 0) a.ceiling[r] = c;
      c = min(c, len - 1);
    }
  }
  if (!ok) {
    for (int j = lane; j <= G; j += kWave) out[j] = -1;
    if (a.mask) {
      for (int k = lane; k < G; k += kWave) a.mask[(size_t)r * G + k] = 0;
    }
    if (lane == 0) {
      a.num_correct[r] = 0;
      a.bonus[r] = -1;
      a.commit[r] = 0;
      if (a.new_seq) a.new_seq[r] = prefix;
      atomicOr(a.meta + 1, DSPARK_DATA_BAD_LENS);
    }
    return;
  }
  const int bon = am[c];
  // column j < gamma holds draft j (lane j's register); column gamma starts at -1
  for (int j = lane; j <= G; j += kWave) out[j] = j == c ? bon : (j < G ? dr : -1);
  if (a.mask) {
    for (int k = lane; k < G; k += kWave) a.mask[(size_t)r * G + k] = k < c ? 1 : 0;
  }
  if (lane == 0) {
    a.num_correct[r] = c;
    a.bonus[r] = bon;
    a.commit[r] = c + 1;
    if (a.new_seq) a.new_seq[r] = prefix + c + 1;
  }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, dspark_dtype dt, int grid, hipStream_t s) {
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(accept_argmax_kernel<DSPARK_BF16>, dim3(grid), dim3(kAccThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(accept_argmax_kernel<DSPARK_F32>, dim3(grid), dim3(kAccThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fgrid = a.B > 0 ? a.B : 1;
  if (a.fixed_rows >= 0) {
    hipLaunchKernelGGL(accept_finalize_kernel<true>, dim3(fgrid), dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL(accept_finalize_kernel<false>, dim3(fgrid), dim3(kWave), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
