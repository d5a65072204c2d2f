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
// Per position k, sts_bin_kernel: each workgroup takes a range of records,
// four threads per record, each on every fourth candidate. For k >= 1 it
// first picks the temperature of position k - 1 from that position's summed
// histograms (the smallest n * ECE, the first candidate on ties; workgroup 0
// records it) and advances the stored survival by it (S_{k-1} =
// RN32(S_{k-2} * sigmoid(z / T*))). Then, for every grid temperature T,
// S = RN32(S_{k-1} * sigmoid(RN32(z_k / T))) is binned into LDS histograms
// (label count and survival sum per bin, Brier sum per T) with LDS atomics,
// and the workgroup adds them into the position's summed histograms with
// 64-bit integer atomics (exact in any order).
// The summed histograms rotate over three buffers: position k adds into
// buffer k % 3, its successor reads it, and workgroup 0 of position k clears
// buffer (k + 1) % 3, which no kernel touches from then until position k + 1
// adds into it. sts_clear_kernel clears buffer 0 first, so the workspace
// needs no initialization. sts_finish_kernel picks the last position's
// temperature and advances the survival by it. The survival lives in two
// buffers used alternately, so a kernel never overwrites what another of its
// threads still has to read.
#include <float.h>
#include <limits.h>

#include "common.h"
#include "sigmoid_cr.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

constexpr double kFx = 0x1p40;

// RN(v * 2^40) as an integer (ties to even), for v in [0, 1] (every value
// binned here is): v * 2^40 + 2^52 in one fused multiply-add is that integer
// plus 2^52, since the doubles in [2^52, 2^53) are exactly the integers, and
// its bits minus those of 2^52 are the integer.
__device__ inline long long fx40(double v) {
  return __double_as_longlong(__fma_rn(v, kFx, 0x1p52)) - __double_as_longlong(0x1p52);
}

// Shared memory of the candidate choice.
struct SelectSmem {
  long long err[DSPARK_STS_MAX_GRID];    // n * ECE * 2^40 per candidate
  long long brier[DSPARK_STS_MAX_GRID];  // n * Brier * 2^40 per candidate
  int t;
};

// Picks the temperature of position kk from its summed histograms h
// ([n_t][2 * nbins + 1]): n * ECE = sum over bins of |labels * 2^40 - survival
// sum|; the smallest wins, the first candidate on ties. Block-wide: with at
// most 16 bins and 16 * n_t threads, thread 16c + b takes bin b of candidate
// c and each 16-lane row sums its candidate; otherwise one (candidate, bin)
// pair per thread and round, summed with LDS atomics. Every thread returns
// the choice. With `record`, the position's results are stored.
__device__ int select_candidate(const StsArgs& a, const long long* h, int kk, bool record,
                                SelectSmem& sm) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int nT = a.n_t, nb = a.nbins, stride = 2 * nb + 1;
  if (nb <= 16 && nT * 16 <= nthr) {
    // one (candidate, bin) per thread, the 16 lanes of a DPP row on one
    // candidate: every load in one round, the row sum by four row shifts
    const int c = tid >> 4, b = tid & 15;
    const bool in = c < nT && b < nb;
    const long long* hc = h + (size_t)(c < nT ? c : 0) * stride;
    const long long lab = in ? hc[b] : 0, sum = in ? hc[nb + b] : 0;
    if (c < nT && b == 0) sm.brier[c] = hc[2 * nb];
    const long long d = lab * (1ll << 40) - sum;
    const long long e = row_incl_scan(d < 0 ? -d : d, 0ll, OpAdd{});
    if (c < nT && b == 15) sm.err[c] = e;
  } else {
    for (int c = tid; c < nT; c += nthr) {
      sm.err[c] = 0;
      sm.brier[c] = h[(size_t)c * stride + 2 * nb];
    }
    __syncthreads();
    for (int i = tid; i < nT * nb; i += nthr) {
      const int c = i / nb, b = i - c * nb;
      const long long d = h[(size_t)c * stride + b] * (1ll << 40) - h[(size_t)c * stride + nb + b];
      if (d != 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&sm.err[c]),
                  (unsigned long long)(d < 0 ? -d : d));
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    long long e = LLONG_MAX;
    int t = INT_MAX;
    for (int c = lane; c < nT; c += kWave) {
      const long long v = sm.err[c];
      if (v < e) e = v, t = c;  // c ascends, so equal errors keep the first
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const long long oe = __shfl_xor(e, off, kWave);
      const int ot = __shfl_xor(t, off, kWave);
      if (oe < e || (oe == e && ot < t)) e = oe, t = ot;
    }
    if (lane == 0) {
      sm.t = t;
      if (record) {
        const double scale = (double)a.N * kFx;
        a.temps[kk] = a.grid[t];
        a.t_index[kk] = t;
        a.ece[kk] = a.N ? (double)e / scale : 0.0;
        a.brier[kk] = a.N ? (double)sm.brier[t] / scale : 0.0;
      }
    }
  }
  if (record && a.ece_grid) {
    for (int c = tid; c < nT; c += nthr) {
      a.ece_grid[(size_t)kk * nT + c] = a.N ? (double)sm.err[c] / ((double)a.N * kFx) : 0.0;
    }
  }
  __syncthreads();
  return sm.t;
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

constexpr int kStsIlp = 2;  // candidates per step of the bin loop (4 was no faster)

__global__ __launch_bounds__(kStsBinThreads) void sts_bin_kernel(StsArgs a, int k) {
  extern __shared__ long long hist[];  // [nT][2 * nbins + 1]: labels, survival sums, Brier
  __shared__ double s_rcp[DSPARK_STS_MAX_GRID];  // RN64(1 / T) per candidate
  __shared__ SelectSmem s_sel;
  const int tid = threadIdx.x;
  const int nb = a.nbins, nT = a.n_t, stride = 2 * nb + 1;
  const size_t hsize = (size_t)nT * stride;
  for (int i = tid; i < nT * stride; i += kStsBinThreads) hist[i] = 0;
  for (int i = tid; i < nT; i += kStsBinThreads) s_rcp[i] = __drcp_rn((double)a.grid[i]);
  if (blockIdx.x == 0) {  // the buffer position k + 1 adds into
    long long* next = a.hists + (size_t)((k + 1) % 3) * hsize;
    for (size_t i = tid; i < hsize; i += kStsBinThreads) next[i] = 0;
  }
  float t_prev = 1.0f;
  if (k > 0) {
    const long long* prev = a.hists + (size_t)((k - 1) % 3) * hsize;
    t_prev = a.grid[select_candidate(a, prev, k - 1, blockIdx.x == 0, s_sel)];
  } else {
    __syncthreads();
  }
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
    // kStsIlp candidates (j, j + 4, ...) per step: their sigmoids' fast
    // paths interleave, and one branch on all the results takes any exact
    // path. Candidate i of a step is used while j + 4 i < nT; past that it
    // repeats the step's first candidate and is dropped.
    for (int j = phase, t = t0; j < nT; j += kStsIlp * kStsPhases) {
      int tc[kStsIlp];
      float x[kStsIlp], c[kStsIlp];
      bool ok[kStsIlp];
#pragma unroll
      for (int i = 0, ti = t; i < kStsIlp; ++i) {
        // t + 4 i (mod nT), kept below nT by one subtraction per step: a
        // candidate past the first is in use only when nT > 4
        tc[i] = j + i * kStsPhases < nT ? ti : t;
        x[i] = div_by_rcp(zk, s_rcp[tc[i]]);
        ti += kStsPhases;
        if (ti >= nT) ti -= nT;
      }
      sigmoid_fast_n<kStsIlp>(x, c, ok);
      bool all_ok = true;
#pragma unroll
      for (int i = 0; i < kStsIlp; ++i) all_ok = all_ok && ok[i];
      if (!all_ok) {
        for (int i = 0; i < kStsIlp; ++i) {
          if (!ok[i]) c[i] = sigmoid_slow(x[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kStsIlp; ++i) {
        if (j + i * kStsPhases >= nT) break;
        const float s = __fmul_rn(sp, c[i]);
        const double sd = s == s ? (double)s : 0.0;  // a NaN survival counts as 0
        int b = (int)(sd * nb);  // sd >= 0 and sd * nb exact: truncation is the floor
        b = b < nb ? b : nb - 1;
        unsigned long long* h = reinterpret_cast<unsigned long long*>(hist + tc[i] * stride);
        if (y) atomicAdd(h + b, 1ull);
        atomicAdd(h + nb + b, (unsigned long long)fx40(sd));
        const double d = sd - (double)y;  // d and d * d each rounded to float64
        atomicAdd(h + 2 * nb, (unsigned long long)fx40(d * d));
      }
#pragma unroll
      for (int i = 0; i < kStsIlp; ++i) {
        t += kStsPhases;
        if (t >= nT) t -= nT;
      }
    }
  }
  __syncthreads();
  unsigned long long* sum = reinterpret_cast<unsigned long long*>(a.hists + (size_t)(k % 3) * hsize);
  for (int i = tid; i < nT * stride; i += kStsBinThreads) {
    const long long v = hist[i];
    if (v != 0) atomicAdd(sum + i, (unsigned long long)v);
  }
}

// Clears summed-histogram buffer 0, which position 0 adds into.
__global__ __launch_bounds__(kStsThreads) void sts_clear_kernel(StsArgs a) {
  const size_t hsize = (size_t)a.n_t * (2 * a.nbins + 1);
  const size_t i = (size_t)blockIdx.x * kStsThreads + threadIdx.x;
  if (i < hsize) a.hists[i] = 0;
}

// Picks the last position's temperature and advances the survival by it.
__global__ __launch_bounds__(kStsThreads) void sts_finish_kernel(StsArgs a) {
  __shared__ SelectSmem s_sel;
  const size_t hsize = (size_t)a.n_t * (2 * a.nbins + 1);
  const int t = select_candidate(a, a.hists + (size_t)((a.gamma - 1) % 3) * hsize, a.gamma - 1,
                                 blockIdx.x == 0, s_sel);
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (a.surv_out && n < a.N) advance_survival(a, a.gamma, n, a.grid[t], true);
}

}  // namespace

hipError_t launch_sts(const StsArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.n_t * (2 * a.nbins + 1) * sizeof(long long);
  const size_t hsize = (size_t)a.n_t * (2 * a.nbins + 1);  // <= 128 * 129
  hipLaunchKernelGGL(sts_clear_kernel, dim3((unsigned)((hsize + kStsThreads - 1) / kStsThreads)),
                     dim3(kStsThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int k = 0; k < a.gamma; ++k) {
    hipLaunchKernelGGL(sts_bin_kernel, dim3(a.n_blocks), dim3(kStsBinThreads), lds, s, a, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int fin = a.surv_out && a.N > 0 ? (a.N + kStsThreads - 1) / kStsThreads : 1;
  hipLaunchKernelGGL(sts_finish_kernel, dim3(fin), dim3(kStsThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
