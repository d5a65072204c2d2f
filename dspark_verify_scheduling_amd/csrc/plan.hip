// Planner kernel: STS confidence -> prefix survival -> global top-b budget
// sweep -> verify_lens, in one workgroup of 1024 threads.
//
// Method sources:
//   "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev)
//     §一: tau(b) = B + sum of the b largest survivals; budget = argmax_b of
//          tau(b) / T(B, B + b); ties go to the earlier position, then the
//          lower request id; ScheduleVerifyLensTopk allocates the budget with
//          min/max_verify_len and survival_eps.
//     §二: runtime STS c_k = sigmoid(z_k / T_k), S_k = prod_{i<=k} c_i.
//     §四: additive cost T(B, M) = bias + alpha(B) + theta(M).
//   "DSpark confidence-scheduled speculative decoding" (charlestar): the
//     prefix-event survival table and the cost model with M = bs + K.
//
// Design for one CU. The whole problem (B*gamma <= 8192 candidates, 64 KB
// of 64-bit keys) fits in LDS, and the step is latency-bound, not
// bandwidth-bound, so one workgroup does it without any global-memory
// round trip:
//   1. thread r walks request r: calibrated confidence, survival (fp32, in
//      order), forced-row tau terms, and one 64-bit key per candidate slot
//      (survival bits | 255-k | 2^24-1-r; 0 for a dropped slot);
//   2. bitonic sort of the keys in LDS, descending, which is exactly
//      (s desc, k asc, r asc) because the keys are unique;
//   3. exact tau by an int64 block scan of survival * 2^40 (nearest), then
//      the fp64 ratio for every b and a (ratio desc, b asc) argmax reduction;
//   4. per-request counts of the first b* keys give verify_lens.
// The arithmetic is written with explicit round-to-nearest intrinsics and
// contraction disabled, so every step has one defined IEEE result.
#include <float.h>

#include "common.h"
#include "sigmoid_cr.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

constexpr int kWaves = kPlanThreads / kWave;
constexpr int kMaxItems = DSPARK_MAX_CANDIDATES / kPlanThreads;  // sorted keys per thread

__device__ inline uint64_t make_key(float s, int k, int r) {
  return ((uint64_t)__float_as_uint(s) << 32) | ((uint64_t)(255 - k) << 24) |
         (uint64_t)(0xFFFFFF - r);
}
__device__ inline float key_s(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }
__device__ inline int key_r(uint64_t key) { return 0xFFFFFF - (int)(key & 0xFFFFFF); }

// survival at the 2^-40 resolution of tau: nearest, ties to even
__device__ inline long long fx40(float s) { return __double2ll_rn((double)s * 0x1p40); }

__device__ inline bool better(double r1, int b1, double r2, int b2) {
  return r1 > r2 || (r1 == r2 && b1 < b2);
}

__device__ void write_fallback(const PlanArgs& a, int flags) {
  for (int r = threadIdx.x; r < a.B; r += kPlanThreads) a.lens[r] = a.lmax;
  if (a.sweep) {
    const int nb = a.B * a.gamma + 1;
    for (int i = threadIdx.x; i < 2 * nb; i += kPlanThreads) a.sweep[i] = __builtin_nan("");
  }
  if (threadIdx.x == 0) {
    a.meta[0] = -1;
    a.meta[1] = -1;
    a.meta[2] = flags;
    a.meta[3] = a.B * a.lmax;
    a.val[0] = __builtin_nan("");
    a.val[1] = __builtin_nan("");
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ uint64_t keys[];  // n_sort keys; later reused as B int counters
  __shared__ long long w64[kWaves + 1];
  __shared__ int w32[kWaves + 1];
  __shared__ double wratio[kWaves];
  __shared__ int wb[kWaves];
  __shared__ int s_flags;

  const int tid = threadIdx.x;
  const int B = a.B, G = a.gamma, lmin = a.lmin, lmax = a.lmax, span = lmax - lmin;
  if (tid == 0) s_flags = 0;
  __syncthreads();

  // ---- 1. survival, forced terms, candidate keys
  long long forced = 0;
  int n_el = 0, bad = 0;
  for (int r = tid; r < B; r += kPlanThreads) {
    float sp = 1.0f;
    for (int k = 1; k <= G; ++k) {
      const float v = a.conf[(size_t)r * G + (k - 1)];
      float s;
      if (a.kind == DSPARK_IN_SURVIVAL) {
        s = v;
        if (!(s >= 0.0f && s <= 1.0f) || (k > 1 && s > sp)) bad = 1;
      } else {
        float c = v;
        if (a.kind == DSPARK_IN_CONF_LOGITS) {
          const float T = a.temps[k - 1];
          if (!(T > 0.0f && T <= FLT_MAX)) bad = 1;
          c = sigmoid_cr(__fdiv_rn(v, T));
        }
        if (!(c >= 0.0f && c <= 1.0f)) bad = 1;
        s = (k == 1) ? c : __fmul_rn(sp, c);
      }
      if (a.surv_out) a.surv_out[(size_t)r * G + (k - 1)] = s;
      if (k < lmin) {
        forced += fx40(s);
      } else if (k < lmax) {
        const bool el = s >= a.eps;
        keys[r * span + (k - lmin)] = el ? make_key(s, k, r) : 0ull;
        n_el += el ? 1 : 0;
      }
      sp = s;
    }
  }
  for (int i = B * span + tid; i < a.n_sort; i += kPlanThreads) keys[i] = 0ull;
  if (bad) atomicOr(&s_flags, DSPARK_DATA_BAD_CONF);
  forced = block_sum<long long, kPlanThreads>(forced, w64);
  n_el = block_sum<int, kPlanThreads>(n_el, w32);
  if (s_flags) {
    write_fallback(a, s_flags);
    return;
  }

  // ---- 2. bitonic sort, descending
  const int n = a.n_sort;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (n >> 1); i += kPlanThreads) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo + j;
        const uint64_t x = keys[lo], y = keys[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? (x < y) : (x > y)) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  // ---- 3. exact tau scan, ratio sweep, argmax
  const int ipt = n >= kPlanThreads ? n / kPlanThreads : 1;
  const int i0 = tid * ipt;
  long long fxv[kMaxItems];
  long long local = 0;
#pragma unroll
  for (int t = 0; t < kMaxItems; ++t) {
    fxv[t] = 0;
    if (t < ipt && i0 + t < n_el) fxv[t] = fx40(key_s(keys[i0 + t]));
    local += fxv[t];
  }
  long long total_fx;
  const long long offset = block_excl_scan<long long, kPlanThreads>(local, w64, &total_fx);
  const long long base = (long long)B * (1ll << 40) + forced;

  const int lo_b = min(max(a.b_lo, 0), n_el);
  const int hi_b = a.b_hi < 0 ? n_el : min(a.b_hi, n_el);
  const double t_fixed = __dadd_rn((double)a.bias, (double)a.alpha[B]);
  const int m0 = B * lmin;

  double tau_v[kMaxItems + 1], ratio_v[kMaxItems + 1];
  double best_r = -1.0;
  int best_b = 0x7fffffff;
  int cost_bad = 0;
  long long run = base + offset;
  // slot 0 of thread 0 is b = 0; slot t + 1 is b = i0 + t + 1
#pragma unroll
  for (int t = 0; t <= kMaxItems; ++t) {
    int b;
    if (t == 0) {
      b = (tid == 0) ? 0 : -1;
    } else {
      run += fxv[t - 1];
      b = (t - 1 < ipt && i0 + t <= n_el) ? i0 + t : -1;
    }
    tau_v[t] = 0.0;
    ratio_v[t] = 0.0;
    if (b < 0) continue;
    const long long tfx = (t == 0) ? base : run;
    const double tau = __ll2double_rn(tfx) * 0x1p-40;
    const double T = __dadd_rn(t_fixed, (double)a.theta[m0 + b]);
    const double ratio = __ddiv_rn(tau, T);
    tau_v[t] = tau;
    ratio_v[t] = ratio;
    if (b >= lo_b && b <= hi_b) {
      if (!(T > 0.0 && T <= DBL_MAX)) cost_bad = 1;
      else if (better(ratio, b, best_r, best_b)) {
        best_r = ratio;
        best_b = b;
      }
    }
  }
  if (cost_bad) atomicOr(&s_flags, DSPARK_DATA_BAD_COST);
  // argmax over the block: (ratio desc, b asc)
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const double orat = __shfl_xor(best_r, off, kWave);
    const int ob = __shfl_xor(best_b, off, kWave);
    if (better(orat, ob, best_r, best_b)) {
      best_r = orat;
      best_b = ob;
    }
  }
  const int lane = lane_id(), wave = tid / kWave;
  if (lane == 0) {
    wratio[wave] = best_r;
    wb[wave] = best_b;
  }
  __syncthreads();
  if (s_flags) {
    write_fallback(a, s_flags);
    return;
  }
  double br = wratio[0];
  int bstar = wb[0];
  for (int w = 1; w < kWaves; ++w) {
    if (better(wratio[w], wb[w], br, bstar)) {
      br = wratio[w];
      bstar = wb[w];
    }
  }

  if (a.sweep) {
    const int nb = B * G + 1;
#pragma unroll
    for (int t = 0; t <= kMaxItems; ++t) {
      const int b = (t == 0) ? (tid == 0 ? 0 : -1) : ((t - 1 < ipt && i0 + t <= n_el) ? i0 + t : -1);
      if (b >= 0) {
        a.sweep[2 * b] = tau_v[t];
        a.sweep[2 * b + 1] = ratio_v[t];
      }
    }
    for (int b = n_el + 1 + tid; b < nb; b += kPlanThreads) {
      a.sweep[2 * b] = __builtin_nan("");
      a.sweep[2 * b + 1] = __builtin_nan("");
    }
  }

  // ---- 4. verify_lens = L_min + #(first b* keys of each request)
  int my_r[kMaxItems];
#pragma unroll
  for (int t = 0; t < kMaxItems; ++t) {
    my_r[t] = (t < ipt && i0 + t < bstar) ? key_r(keys[i0 + t]) : -1;
  }
  __syncthreads();
  int* cnt = reinterpret_cast<int*>(keys);
  for (int r = tid; r < B; r += kPlanThreads) cnt[r] = 0;
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kMaxItems; ++t) {
    if (my_r[t] >= 0) atomicAdd(&cnt[my_r[t]], 1);
  }
  __syncthreads();
  for (int r = tid; r < B; r += kPlanThreads) a.lens[r] = lmin + cnt[r];
  if (tid == 0) {
    a.meta[0] = bstar;
    a.meta[1] = n_el;
    a.meta[2] = 0;
    a.meta[3] = m0 + bstar;
  }
  // tau(b*) and ratio(b*) from the thread that owns b*
#pragma unroll
  for (int t = 0; t <= kMaxItems; ++t) {
    const int b = (t == 0) ? (tid == 0 ? 0 : -1) : ((t - 1 < ipt && i0 + t <= n_el) ? i0 + t : -1);
    if (b == bstar) {
      a.val[0] = tau_v[t];
      a.val[1] = ratio_v[t];
    }
  }
}

}  // namespace

size_t plan_lds_bytes(int B, int n_sort) {
  size_t k = (size_t)n_sort * sizeof(uint64_t);
  size_t c = (size_t)B * sizeof(int);
  return k > c ? k : c;
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const size_t lds = plan_lds_bytes(a.B, a.n_sort);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace dspark
