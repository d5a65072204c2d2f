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
//   sts_bin_kernel: each workgroup takes a range of records, four threads per
//     record, each on every fourth candidate. For k >= 1 it first picks the
//     temperature of position k - 1 (the smallest summed error, the first
//     candidate on ties; workgroup 0 records it) and advances the stored
//     survival by it (S_{k-1} = RN32(S_{k-2} * sigmoid(z / T*))). Then, for
//     every grid temperature T, S = RN32(S_{k-1} * sigmoid(RN32(z_k / T)))
//     is binned into LDS histograms (label count and survival sum per bin,
//     Brier sum per T) with LDS atomics, and the workgroup writes its
//     histograms to its slot of the workspace (no cross-workgroup atomics).
//   sts_reduce_kernel: one workgroup per candidate sums the slots and forms
//     n * ECE and n * Brier for it.
// sts_finish_kernel picks the last position's temperature and advances the
// survival by it. The survival lives in two buffers used alternately, so a
// kernel never overwrites what another of its threads still has to read.
#include <float.h>
#include <limits.h>

#include "common.h"
#include "sigmoid_cr.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

constexpr double kFx = 0x1p40;

__device__ inline long long fx40(double v) { return __double2ll_rn(v * kFx); }

// Picks the temperature of position kk from the summed errors (one wave):
// the smallest n * ECE, the first candidate on ties. Every lane returns it;
// with `record` set, lane 0 also stores the position's results.
__device__ int select_candidate(const StsArgs& a, int kk, bool record) {
  const int lane = lane_id();
  const long long* err = a.err_fx + (size_t)kk * a.n_t;
  long long e = LLONG_MAX;
  int t = INT_MAX;
  for (int c = lane; c < a.n_t; c += kWave) {
    const long long v = err[c];
    if (v < e) e = v, t = c;  // c ascends, so equal errors keep the first
  }
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const long long oe = __shfl_xor(e, off, kWave);
    const int ot = __shfl_xor(t, off, kWave);
    if (oe < e || (oe == e && ot < t)) e = oe, t = ot;
  }
  if (record && lane == 0) {
    const double scale = (double)a.N * kFx;
    a.temps[kk] = a.grid[t];
    a.t_index[kk] = t;
    a.ece[kk] = a.N ? (double)e / scale : 0.0;
    a.brier[kk] = a.N ? (double)a.brier_fx[(size_t)kk * a.n_t + t] / scale : 0.0;
  }
  return t;
}

// S_{k-1} for record n: 1 at k = 0, else S_{k-2} times the calibrated
// confidence of position k - 1 at its chosen temperature. The writer stores
// it (buffer (k - 1) & 1, and the survival output).
__device__ inline float advance_survival(const StsArgs& a, int k, int n, float t_prev, bool writer) {
  if (k == 0) return 1.0f;
  const float c = sigmoid_cr(__fdiv_rn(a.z[(size_t)n * a.gamma + (k - 1)], t_prev));
  const float s0 = k == 1 ? 1.0f : a.s_work[k & 1][n];
  const float s = __fmul_rn(s0, c);
  if (writer) {
    a.s_work[(k - 1) & 1][n] = s;
    if (a.surv_out) a.surv_out[(size_t)n * a.gamma + (k - 1)] = s;
  }
  return s;
}

// RN32(z / T) as RN32(RN64(z * RN64(1 / T))), for any float32 z and T: the
// double value is within 2^-52 (relative) of z / T, while z / T is never a
// float32 rounding midpoint and is always more than 2^-49 (relative) away
// from one. (A midpoint has at most 25 significant bits and is odd in its
// last one; times T it has more bits than z, so z - M * T is a nonzero
// multiple of 2^e with 2^e > |z| * 2^-49.) Zeros, infinities and NaNs give
// the quotient's own special value.
__device__ inline float div_by_rcp(double z, double rcp_t) {
  return __double2float_rn(__dmul_rn(z, rcp_t));
}

__global__ __launch_bounds__(kStsBinThreads) void sts_bin_kernel(StsArgs a, int k) {
  extern __shared__ long long hist[];  // [nT][2 * nbins + 1]: labels, survival sums, Brier
  __shared__ double s_rcp[DSPARK_STS_MAX_GRID];  // RN64(1 / T) per candidate
  __shared__ int s_prev;
  const int tid = threadIdx.x;
  const int nb = a.nbins, nT = a.n_t, stride = 2 * nb + 1;
  for (int i = tid; i < nT * stride; i += kStsBinThreads) hist[i] = 0;
  for (int i = tid; i < nT; i += kStsBinThreads) s_rcp[i] = __drcp_rn((double)a.grid[i]);
  if (k > 0 && tid < kWave) {
    const int t = select_candidate(a, k - 1, blockIdx.x == 0);
    if (tid == 0) s_prev = t;
  }
  __syncthreads();
  const float t_prev = k > 0 ? a.grid[s_prev] : 1.0f;
  const int slot = tid % kStsPass, phase = tid / kStsPass;  // phase is wave-uniform
  // a lane visits candidates (lane + phase + 4 i) mod nT, so the four phases
  // cover every candidate once and the lanes of a wave start on different rows
  const int t0 = (lane_id() + phase) % nT;
  const int r0 = blockIdx.x * a.per_block;
  const int r1 = min(r0 + a.per_block, a.N);
  for (int n = r0 + slot; n < r1; n += kStsPass) {
    const float sp = advance_survival(a, k, n, t_prev, phase == 0);
    const double zk = (double)a.z[(size_t)n * a.gamma + k];
    const unsigned long long y = a.labels[(size_t)n * a.gamma + k] ? 1ull : 0ull;
    for (int j = phase, t = t0; j < nT; j += kStsPhases) {
      const float s = __fmul_rn(sp, sigmoid_cr(div_by_rcp(zk, s_rcp[t])));
      const double sd = s == s ? (double)s : 0.0;  // a NaN survival counts as 0
      int b = (int)floor(sd * nb);
      b = b < nb ? b : nb - 1;
      unsigned long long* h = reinterpret_cast<unsigned long long*>(hist + t * stride);
      if (y) atomicAdd(h + b, 1ull);
      atomicAdd(h + nb + b, (unsigned long long)fx40(sd));
      const double d = sd - (double)y;  // exact, and so is d * d
      atomicAdd(h + 2 * nb, (unsigned long long)fx40(d * d));
      t += kStsPhases;
      if (t >= nT) t -= nT;  // once past the end only when nT > 4: then t < nT again
    }
  }
  __syncthreads();
  long long* out = a.partials + (size_t)blockIdx.x * nT * stride;
  for (int i = tid; i < nT * stride; i += kStsBinThreads) out[i] = hist[i];
}

// Workgroup t: sums candidate t's histogram slots over the bin workgroups.
// Thread (q, c) adds column c of slots q, q + Q, q + 2Q, ... in a register.
__global__ __launch_bounds__(kStsReduceThreads) void sts_reduce_kernel(StsArgs a, int k) {
  __shared__ long long col[2 * DSPARK_STS_MAX_BINS + 1];
  __shared__ long long s_err;
  const int tid = threadIdx.x, t = blockIdx.x;
  const int nb = a.nbins, nT = a.n_t, stride = 2 * nb + 1;
  for (int c = tid; c < stride; c += kStsReduceThreads) col[c] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const int Q = kStsReduceThreads / stride;  // >= 7: stride <= 2 * 64 + 1
  if (tid < Q * stride) {
    const int q = tid / stride, c = tid - q * stride;
    const long long* p = a.partials + ((size_t)q * nT + t) * stride + c;
    const size_t step = (size_t)Q * nT * stride;
    long long acc = 0;
#pragma unroll 8
    for (int g = q; g < a.n_blocks; g += Q, p += step) acc += *p;
    atomicAdd(reinterpret_cast<unsigned long long*>(col + c), (unsigned long long)acc);
  }
  __syncthreads();
  for (int b = tid; b < nb; b += kStsReduceThreads) {
    const long long diff = col[b] * (1ll << 40) - col[nb + b];
    atomicAdd(reinterpret_cast<unsigned long long*>(&s_err),
              (unsigned long long)(diff < 0 ? -diff : diff));
  }
  __syncthreads();
  if (tid == 0) {
    a.err_fx[(size_t)k * nT + t] = s_err;
    a.brier_fx[(size_t)k * nT + t] = col[2 * nb];
    if (a.ece_grid) a.ece_grid[(size_t)k * nT + t] = a.N ? (double)s_err / ((double)a.N * kFx) : 0.0;
  }
}

// Picks the last position's temperature and advances the survival by it.
__global__ __launch_bounds__(kStsThreads) void sts_finish_kernel(StsArgs a) {
  __shared__ int s_prev;
  if (threadIdx.x < kWave) {
    const int t = select_candidate(a, a.gamma - 1, blockIdx.x == 0);
    if (threadIdx.x == 0) s_prev = t;
  }
  __syncthreads();
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (a.surv_out && n < a.N) advance_survival(a, a.gamma, n, a.grid[s_prev], true);
}

}  // namespace

hipError_t launch_sts(const StsArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.n_t * (2 * a.nbins + 1) * sizeof(long long);
  for (int k = 0; k < a.gamma; ++k) {
    hipLaunchKernelGGL(sts_bin_kernel, dim3(a.n_blocks), dim3(kStsBinThreads), lds, s, a, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sts_reduce_kernel, dim3(a.n_t), dim3(kStsReduceThreads), 0, s, a, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int fin = a.surv_out && a.N > 0 ? (a.N + kStsThreads - 1) / kStsThreads : 1;
  hipLaunchKernelGGL(sts_finish_kernel, dim3(fin), dim3(kStsThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
