// Sequential temperature scaling (STS) fitter: one temperature per draft
// position, chosen from a grid by expected calibration error.
//
// Method sources: "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §二 (the
// fitter searches a positive temperature per position, in order, keeping the
// cumulative survival already fitted for the earlier positions, and keeps the
// candidate with the lower ECE against the greedy prefix label) and "DSpark
// confidence-scheduled speculative decoding" (charlestar), the calibration
// section (ECE = sum_b |I_b| / n * |acc(I_b) - conf(I_b)|; a position's label
// only has meaning given that the earlier positions survived).
//
// Exact arithmetic. n * ECE = sum_b |L_b - C_b| with L_b the labels and C_b
// the survivals of bin b; each survival enters C_b at 2^-40 resolution
// (nearest), so every sum is an int64 and the argmin over the grid is an
// exact, order-independent decision. Brier terms likewise.
//
// Per position k:
//   sts_bin_kernel: each workgroup takes a range of records. For k >= 1 it
//     first advances the stored survival by the temperature chosen for k - 1
//     (S_{k-1} = RN32(S_{k-2} * sigmoid(z / T*))) and writes it out. Then, for
//     every grid temperature T, S = RN32(S_{k-1} * sigmoid(RN32(z_k / T)))
//     is binned into LDS histograms (label count and survival sum per bin,
//     Brier sum per T) with LDS atomics, and the workgroup writes its
//     histograms to its slot of the workspace (no cross-workgroup atomics).
//   sts_select_kernel: one workgroup sums the slots per T, forms n * ECE,
//     picks the smallest (the first T on ties) and records the result.
// sts_finish_kernel advances the survival for the last position.
#include <float.h>

#include "common.h"
#include "sigmoid_cr.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

constexpr double kFx = 0x1p40;

__device__ inline long long fx40(double v) { return __double2ll_rn(v * kFx); }

// Survival of the previous position: 1 at k = 0, else advanced in place.
__device__ inline float prev_survival(const StsArgs& a, int k, int n) {
  if (k == 0) return 1.0f;
  const float t = a.chosen_t[k - 1];
  const float c = sigmoid_cr(__fdiv_rn(a.z[(size_t)n * a.gamma + (k - 1)], t));
  const float s0 = k == 1 ? 1.0f : a.s_work[n];
  const float s = __fmul_rn(s0, c);
  a.s_work[n] = s;
  if (a.surv_out) a.surv_out[(size_t)n * a.gamma + (k - 1)] = s;
  return s;
}

__global__ __launch_bounds__(kStsThreads) void sts_bin_kernel(StsArgs a, int k) {
  extern __shared__ long long hist[];  // [nT][2 * nbins + 1]: labels, survival sums, Brier
  const int tid = threadIdx.x;
  const int nb = a.nbins, nT = a.n_t, stride = 2 * nb + 1;
  for (int i = tid; i < nT * stride; i += kStsThreads) hist[i] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * a.per_block;
  const int r1 = min(r0 + a.per_block, a.N);
  for (int n = r0 + tid; n < r1; n += kStsThreads) {
    const float sp = prev_survival(a, k, n);
    const float zk = a.z[(size_t)n * a.gamma + k];
    const int y = a.labels[(size_t)n * a.gamma + k] ? 1 : 0;
    // lanes start at different candidates so their LDS atomics hit different rows
    for (int tt = 0, t = lane_id() % nT; tt < nT; ++tt, t = t + 1 < nT ? t + 1 : 0) {
      const float s = __fmul_rn(sp, sigmoid_cr(__fdiv_rn(zk, a.grid[t])));
      const double sd = s == s ? (double)s : 0.0;  // a NaN survival counts as 0
      int b = (int)floor(sd * nb);
      b = b < nb ? b : nb - 1;
      long long* h = hist + t * stride;
      if (y) atomicAdd(reinterpret_cast<unsigned long long*>(h + b), 1ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(h + nb + b), (unsigned long long)fx40(sd));
      const double d = sd - (double)y;  // exact, and so is d * d
      atomicAdd(reinterpret_cast<unsigned long long*>(h + 2 * nb), (unsigned long long)fx40(d * d));
    }
  }
  __syncthreads();
  long long* out = a.partials + (size_t)blockIdx.x * nT * stride;
  for (int i = tid; i < nT * stride; i += kStsThreads) out[i] = hist[i];
}

__global__ __launch_bounds__(kStsThreads) void sts_select_kernel(StsArgs a, int k) {
  __shared__ long long s_err[DSPARK_STS_MAX_GRID];
  __shared__ long long s_brier[DSPARK_STS_MAX_GRID];
  const int tid = threadIdx.x;
  const int nb = a.nbins, nT = a.n_t, stride = 2 * nb + 1;
  for (int t = tid; t < nT; t += kStsThreads) s_err[t] = 0;
  __syncthreads();
  // one (T, bin) item per thread at a time; the last column of a T is its Brier sum
  for (int p = tid; p < nT * (nb + 1); p += kStsThreads) {
    const int t = p / (nb + 1);
    const int b = p - t * (nb + 1);
    if (b < nb) {
      long long lab = 0, conf = 0;
      for (int g = 0; g < a.n_blocks; ++g) {
        const long long* h = a.partials + ((size_t)g * nT + t) * stride;
        lab += h[b];
        conf += h[nb + b];
      }
      const long long diff = lab * (1ll << 40) - conf;
      atomicAdd(reinterpret_cast<unsigned long long*>(s_err + t),
                (unsigned long long)(diff < 0 ? -diff : diff));
    } else {
      long long brier = 0;
      for (int g = 0; g < a.n_blocks; ++g) brier += a.partials[((size_t)g * nT + t) * stride + 2 * nb];
      s_brier[t] = brier;
    }
  }
  __syncthreads();
  const double scale = (double)a.N * kFx;
  if (a.ece_grid) {
    for (int t = tid; t < nT; t += kStsThreads) {
      a.ece_grid[(size_t)k * nT + t] = a.N ? (double)s_err[t] / scale : 0.0;
    }
  }
  if (tid == 0) {
    int best = 0;
    for (int t = 1; t < nT; ++t) {
      if (s_err[t] < s_err[best]) best = t;
    }
    a.chosen_t[k] = a.grid[best];
    a.temps[k] = a.grid[best];
    a.t_index[k] = best;
    a.ece[k] = a.N ? (double)s_err[best] / scale : 0.0;
    a.brier[k] = a.N ? (double)s_brier[best] / scale : 0.0;
  }
}

// Advances the survival by the temperature chosen for the last position.
__global__ __launch_bounds__(kStsThreads) void sts_finish_kernel(StsArgs a) {
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (n < a.N) prev_survival(a, a.gamma, n);
}

}  // namespace

hipError_t launch_sts(const StsArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.n_t * (2 * a.nbins + 1) * sizeof(long long);
  for (int k = 0; k < a.gamma; ++k) {
    hipLaunchKernelGGL(sts_bin_kernel, dim3(a.n_blocks), dim3(kStsThreads), lds, s, a, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sts_select_kernel, dim3(1), dim3(kStsThreads), 0, s, a, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.N > 0) {
    hipLaunchKernelGGL(sts_finish_kernel, dim3((a.N + kStsThreads - 1) / kStsThreads),
                       dim3(kStsThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
