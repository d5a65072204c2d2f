// Planner kernel: STS confidence -> prefix survival -> global top-b budget
// sweep -> verify_lens, in one workgroup of 1024 threads; optionally followed
// in the same workgroup by the compact layout (cu_seqlens, packed rows, tier).
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
// of 64-bit keys) fits in LDS and the step is latency-bound, so one
// workgroup does it without any global-memory round trip:
//   1. every (request, position) confidence is calibrated in parallel; then
//      thread r walks request r for the survival product (fp32, in order),
//      the forced-row tau terms, and one 64-bit key per candidate slot
//      (survival bits | 255-k | 2^24-1-r; 0 for a dropped slot). The cost
//      entries the sweep will need are loaded at kernel start.
//   2. the global order (s desc, k asc, r asc) is the descending order of
//      the unique keys. A bucket sort on the survival bits over the observed
//      range [min, max] (about one key per bucket) places every key with one
//      LDS atomic, a scan of the bucket counts and an exact rank among its
//      bucket's few members: three or four barriers and O(n) work. If a bucket holds
//      more than 32 keys (many equal survivals), the keys are instead merged
//      from the per-request runs, which are already descending, pairwise in
//      ceil(log2 B) rounds of merge path. Both give the same order.
//   3. (sorted positions spread over all 16 waves)
//      exact tau by an int64 block scan of survival * 2^40 (nearest), the
//      fp64 ratio for every b, and a (ratio desc, b asc) argmax reduction;
//   4. per-request counts of the first b* keys give verify_lens;
//   5. (fused variant) the exclusive scan, tier and front-packed rows.
// Variants ("DSpark 自适应 Verify 怎样分配候选预算" §一, §四, §五): the
// objective tau(b) * SPS(M) with SPS read by floor lookup from a table of
// probe points (kept in LDS; each thread walks it along its budgets), and
// graph-tier alignment, which extends the executed budget with the next
// sorted candidates up to the tier the chosen budget already pays for.
// The arithmetic uses explicit round-to-nearest intrinsics with contraction
// disabled, so every step has one defined IEEE result.
#include <float.h>

#include "common.h"
#include "pack_dev.h"
#include "sigmoid_cr.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

constexpr int kWaves = kPlanThreads / kWave;
constexpr int kMaxItems = DSPARK_MAX_CANDIDATES / kPlanThreads;  // keys per thread, at most
static_assert(kMaxItems == 8, "item counts 1, 2, 4, 8 cover every B * gamma");
constexpr int kLgMinBuckets = 6, kLgMaxBuckets = 12;
constexpr int kMaxBuckets = 1 << kLgMaxBuckets;
constexpr int kMaxBucketFill = 32;  // beyond this the bucket rank loop gives way to merging

__device__ inline uint64_t make_key(float s, int k, int r) {
  return ((uint64_t)__float_as_uint(s) << 32) | ((uint64_t)(255 - k) << 24) |
         (uint64_t)(0xFFFFFF - r);
}
__device__ inline float key_s(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }
__device__ inline int key_r(uint64_t key) { return 0xFFFFFF - (int)(key & 0xFFFFFF); }

// survival at the 2^-40 resolution of tau: nearest, ties to even, for s in
// [0, 1] (any other value sends the planner to its fallback, which discards
// it). s * 2^40 + 2^52 in one fused multiply-add is that integer plus 2^52,
// since the doubles in [2^52, 2^53) are exactly the integers; its bits minus
// those of 2^52 are the integer.
__device__ inline long long fx40(float s) {
  return __double_as_longlong(__fma_rn((double)s, 0x1p40, 0x1p52)) -
         __double_as_longlong(0x1p52);
}

__device__ inline bool better(double r1, int b1, double r2, int b2) {
  return r1 > r2 || (r1 == r2 && b1 < b2);
}

// The cross-wave steps below read one per-wave partial per lane of a 16-lane
// row (lane l takes wave l & 15's), so every row holds all of them and four
// row shifts combine them.
static_assert(kWaves == 16, "one per-wave partial per lane of a 16-lane row");

struct OpMaxD {
  __device__ double operator()(double x, double y) const { return __builtin_fmax(x, y); }
};

// The (ratio desc, b asc) maximum of one value per lane over the lanes whose
// bit is set in `lanes`, where the lane order is the order of b (each lane's
// budgets lie below the next lane's): the maximum ratio by DPP steps, then
// the b of the lowest lane holding it, which is the smallest b among equal
// ratios. A lane's "none" is (-1, INT_MAX); every real ratio is >= 0 and
// none is NaN, so the maximum is one of the lanes' values, bit for bit.
// Wave-uniform results.
template <bool ROW>
__device__ inline void lane_argmax(double r, int b, unsigned long long lanes, double& best_r,
                                   int& best_b) {
  best_r = ROW ? read_lane(row_incl_scan(r, -1.0, OpMaxD{}), 15)
               : read_lane(wave_incl_scan_op(r, -1.0, OpMaxD{}), kWave - 1);
  const unsigned long long hit = __ballot(r == best_r) & lanes;
  best_b = __builtin_amdgcn_readlane(b, (int)__builtin_ctzll(hit));
}

// Number of keys in the descending run d[0, len) greater than `key`
// (strict = true) or greater than or equal to it (strict = false).
template <bool STRICT>
__device__ inline int count_above(const uint64_t* d, int len, uint64_t key) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const bool above = STRICT ? d[mid] > key : d[mid] >= key;
    if (above) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Merges the descending runs src[i*L, (i+1)*L) (the last one may be
// shorter) pairwise until one run remains, ping-ponging between src and dst.
// Each key finds its place by one binary search in the partner run: a key of
// the first run of a pair goes after the partner's strictly greater keys, a
// key of the second run after the partner's greater-or-equal keys, so equal
// keys (the zero padding) keep a consistent order and every position is
// written once. Returns the buffer that holds the merged run. Block-wide.
__device__ uint64_t* merge_runs(uint64_t* src, uint64_t* dst, int n, int L) {
  for (int runs = (n + L - 1) / L; runs > 1; runs = (runs + 1) >> 1, L <<= 1) {
    for (int g = threadIdx.x; g < n; g += kPlanThreads) {
      const uint64_t key = src[g];
      const int i = g / L;
      const int off = g - i * L;
      int pos;
      if (i & 1) {
        pos = (i - 1) * L + off + count_above<false>(src + (i - 1) * L, L, key);
      } else {
        const int b0 = (i + 1) * L;
        const int blen = min(L, max(0, n - b0));
        pos = i * L + off + count_above<true>(src + b0, blen, key);
      }
      dst[pos] = key;
    }
    __syncthreads();
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  return src;
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

// Static window for every request: the fallback for bad data (and, in the
// fused variant, its packed layout).
// Pack inputs prefetched per thread by the fused kernel (3 slots cover
// B * (gamma + 1) <= 3072 verify slots, e.g. B = 256 at gamma = 8).
constexpr int kPackPrefetch = 3;
using PlanPrefetch = PackPrefetch<kPlanThreads, kPackPrefetch>;

template <bool PACK>
__device__ void fallback(const PlanArgs& a, const PackArgs& p, int flags, uint64_t* lds, int* w32,
                         int tier_lane, const PlanPrefetch* pre) {
  write_fallback(a, flags);
  if (PACK) {
    int32_t* lens = reinterpret_cast<int32_t*>(lds);
    for (int r = threadIdx.x; r < a.B; r += kPlanThreads) lens[r] = a.lmax;
    __syncthreads();
    pack_block<kPlanThreads, kPackPrefetch>(p, lens, lens + a.B, w32, tier_lane, 0, pre);
  }
}

// LDS layout of the planner, in bytes (all offsets 8-byte aligned):
//   [0, K)        keys: one 64-bit key per candidate slot (n_keys slots)
//   [K, K + X)    phase 1: calibrated confidences (B * gamma floats);
//                 then the second key buffer (n_keys) followed by the bucket
//                 counts (kMaxBuckets + 1 ints)
// The fused pack reuses [0, (2B + 1) * 4) at the end.
__host__ __device__ inline size_t plan_x_bytes(int B, int gamma, int n_keys) {
  const size_t c = (size_t)B * gamma * sizeof(float);
  const size_t k = (size_t)n_keys * sizeof(uint64_t) + (size_t)(kMaxBuckets + 1) * sizeof(int);
  return c > k ? c : k;
}

// ITEMS = the items (confidences, keys, sorted positions) each thread holds
// at most: a power of two >= B * gamma / 1024, so that the per-item loops
// are unrolled over live items only.
template <bool PACK, int ITEMS>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a, PackArgs p) {
  extern __shared__ uint64_t lds[];
  __shared__ long long w64[kWaves + 1];
  __shared__ int w32[kWaves + 1];
  __shared__ double wratio[kWaves];
  __shared__ int wb[kWaves];
  __shared__ int s_flags;
  __shared__ unsigned int wmin[kWaves], wmax[kWaves];
  __shared__ int wbad[kWaves];
  __shared__ int s_maxb;
  __shared__ int s_pm[DSPARK_MAX_SPS_PROBES];    // SPS probe totals
  __shared__ float s_ps[DSPARK_MAX_SPS_PROBES];  // SPS at each probe

  const int tid = threadIdx.x;
  const int B = a.B, G = a.gamma, lmin = a.lmin, lmax = a.lmax, span = lmax - lmin;
  const int n_keys = B * span;
  const int ipt = (n_keys + kPlanThreads - 1) / kPlanThreads;  // sorted positions per thread
  const int base_i = tid * ipt;
  const int m0 = B * lmin;
  uint64_t* keys = lds;
  unsigned char* xreg = reinterpret_cast<unsigned char*>(lds + n_keys);
  float* conf_c = reinterpret_cast<float*>(xreg);
  uint64_t* aux = reinterpret_cast<uint64_t*>(xreg);
  int* bucket = reinterpret_cast<int*>(xreg + (size_t)n_keys * sizeof(uint64_t));
  if (tid == 0) {
    s_flags = 0;
    s_maxb = 0;
  }

  // this thread's confidences (and their temperatures) first: the
  // calibration waits for them, not for the loads issued after them
  const SmallDiv per_req(G);  // B * gamma <= 8192
  const bool logits = a.kind == DSPARK_IN_CONF_LOGITS;
  float cin[ITEMS], tin[ITEMS];
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    const int idx = tid + e * kPlanThreads;
    cin[e] = 0.0f;
    tin[e] = 1.0f;
    if (idx < B * G) {
      cin[e] = a.conf[idx];
      if (logits) tin[e] = a.temps[idx - per_req.quo(idx) * G];
    }
  }

  PlanPrefetch pre;
  int tier_lane = 0;
  if (PACK) {
    pre.load(p);
    tier_lane = load_tier_lane(p);
  }
  // cost entries of the budgets this thread will evaluate: b = base_i + e + 1
  const bool sps_mode = a.cost_mode == DSPARK_COST_SPS1D;
  float th[ITEMS];
  float th0 = 0.0f, alpha_b = 0.0f;
  if (sps_mode) {
    for (int i = tid; i < a.sps_len; i += kPlanThreads) {
      s_pm[i] = a.sps_m[i];
      s_ps[i] = a.sps[i];
    }
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) th[e] = 0.0f;
  } else {
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) {
      const int m = m0 + base_i + e + 1;
      th[e] = (e < ipt && base_i + e < n_keys && m < a.theta_len) ? a.theta[m] : 0.0f;
    }
    th0 = a.theta[m0];
    alpha_b = a.alpha[B];
  }

  // ---- 1a. calibrated confidence of every (request, position), in parallel
  int bad = 0;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    const int idx = tid + e * kPlanThreads;
    if (idx < B * G) {
      const float v = cin[e];
      float c = v;
      if (logits) {
        const float T = tin[e];
        if (!(T > 0.0f && T <= FLT_MAX)) bad = 1;
        c = sigmoid_cr(__fdiv_rn(v, T));
      }
      if (!(c >= 0.0f && c <= 1.0f)) bad = 1;
      conf_c[idx] = c;
    }
  }
  __syncthreads();
  // The bucket counts of the sort lie past the confidences when B * gamma
  // floats fit in the key buffer's bytes: then they are cleared here, and the
  // reduction's barrier below orders the clear before the counting.
  const bool early_clear = (size_t)B * G * sizeof(float) <= (size_t)n_keys * sizeof(uint64_t);
  if (early_clear) {
    for (int i = tid; i <= kMaxBuckets; i += kPlanThreads) bucket[i] = 0;
  }

  // ---- 1b. survival, forced terms, candidate keys: one thread per
  // (request, position). Thread (r, k) forms c_1 * ... * c_k itself, left to
  // right in fp32: the same operations in the same order as a running
  // product, so the same bits, without a serial walk along each request.
  long long forced = 0;
  int n_el = 0;
  unsigned int smin = 0xFFFFFFFFu, smax = 0u;
  auto emit = [&](int idx, int r, int k, float s) {
    if (a.surv_out) a.surv_out[idx] = s;
    if (k < lmin) {
      forced += fx40(s);
    } else if (k < lmax) {
      const bool el = s >= a.eps;
      // -0 ranks with +0 (the order is by value): the key takes +0's bits
      const float sk = s == 0.0f ? 0.0f : s;
      keys[r * span + (k - lmin)] = el ? make_key(sk, k, r) : 0ull;
      if (el) {
        ++n_el;
        const unsigned int sb = __float_as_uint(sk);
        smin = min(smin, sb);
        smax = max(smax, sb);
      }
    }
  };
  if (a.kind != DSPARK_IN_SURVIVAL && G <= 9 && ITEMS <= 4) {
    // at most 8 factors after the first: every item's reads (clamped to the
    // request's last position; an item past B * gamma reads request 0 and is
    // dropped) are issued before the first multiply, and a factor past the
    // item's own position is never multiplied, so each product keeps its
    // left-to-right order
    float f[ITEMS][9];
    int kk[ITEMS], rr[ITEMS];
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) {
      const int idx = tid + e * kPlanThreads;
      const int r = idx < B * G ? per_req.quo(idx) : 0;
      rr[e] = r;
      kk[e] = idx - r * G + 1;
      const float* cr = conf_c + r * G;
#pragma unroll
      for (int j = 0; j < 9; ++j) f[e][j] = cr[min(j, G - 1)];
    }
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) {
      const int idx = tid + e * kPlanThreads;
      if (idx < B * G) {
        float s = f[e][0];
#pragma unroll
        for (int j = 1; j < 9; ++j) s = j < kk[e] ? __fmul_rn(s, f[e][j]) : s;
        emit(idx, rr[e], kk[e], s);
      }
    }
  } else {
    for (int idx = tid; idx < B * G; idx += kPlanThreads) {
      const int r = per_req.quo(idx);
      const int k = idx - r * G + 1;
      const float* cr = conf_c + r * G;
      float s = cr[0];
      if (a.kind == DSPARK_IN_SURVIVAL) {
        s = cr[k - 1];
        if (k > 1 && s > cr[k - 2]) bad = 1;
      } else {
        // factors 1 .. k-1 in batches of 8, each batch's LDS reads issued
        // before its first multiply; a read past the request's last position
        // is never multiplied, so the product keeps its left-to-right order
        for (int i0 = 1; i0 < k; i0 += 8) {
          float f[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = cr[min(i0 + j, G - 1)];
#pragma unroll
          for (int j = 0; j < 8; ++j) s = i0 + j < k ? __fmul_rn(s, f[j]) : s;
        }
      }
      emit(idx, r, k, s);
    }
  }
  // SPS probes must be strictly ascending (bit 1 of `bad`: a cost error,
  // reported after any confidence error)
  if (sps_mode) {
    for (int i = tid + 1; i < a.sps_len; i += kPlanThreads) {
      if (s_pm[i] <= s_pm[i - 1]) bad |= 2;
    }
  }
  // one block reduction for the five quantities: per-wave DPP reductions,
  // then every wave combines the 16 per-wave partials. The flags go through
  // ballots, and the forced sum is reduced only when positions are forced.
  {
    const int lane = lane_id(), wave = tid / kWave;
    auto umin = [](unsigned int x, unsigned int y) { return min(x, y); };
    auto umax = [](unsigned int x, unsigned int y) { return max(x, y); };
    auto flags_of = [](int v) {
      return (__ballot((v & 1) != 0) ? 1 : 0) | (__ballot((v & 2) != 0) ? 2 : 0);
    };
    const bool any_forced = lmin > 1;
    if (any_forced) forced = wave_incl_scan_op(forced, 0ll, OpAdd{});
    n_el = wave_incl_scan_op(n_el, 0, OpAdd{});
    smin = wave_incl_scan_op(smin, 0xFFFFFFFFu, umin);
    smax = wave_incl_scan_op(smax, 0u, umax);
    const int wflags = flags_of(bad);
    if (lane == kWave - 1) {
      w64[wave] = forced;
      w32[wave] = n_el;
      wmin[wave] = smin;
      wmax[wave] = smax;
      wbad[wave] = wflags;
    }
    __syncthreads();
    const int l = lane & 15;
    const int n2 = w32[l], b2 = wbad[l];
    const unsigned int mn2 = wmin[l], mx2 = wmax[l];
    if (any_forced) forced = read_lane(row_incl_scan(w64[l], 0ll, OpAdd{}), 15);
    n_el = read_lane(row_incl_scan(n2, 0, OpAdd{}), 15);
    smin = read_lane(row_incl_scan(mn2, 0xFFFFFFFFu, umin), 15);
    smax = read_lane(row_incl_scan(mx2, 0u, umax), 15);
    bad = flags_of(b2);  // every row holds all 16 waves' flags
    // no closing barrier: w32 is written again only after the counting
    // barrier of the sort (or the fallback's barrier); the others never
  }
  if (bad) {
    fallback<PACK>(a, p, (bad & 1) ? DSPARK_DATA_BAD_CONF : DSPARK_DATA_BAD_COST, lds, w32,
                   tier_lane, &pre);
    return;
  }

  // ---- 2. order the candidates by key, descending: bucket sort on the
  // survival bits over [smin, smax], exact rank inside each bucket
  const uint64_t* sorted = keys;
  if (n_el > 0) {
    const unsigned int hi = smax, range = smax - smin;
    // nb = the power of two in [64, 4096] nearest above n_el; shift = the
    // least s with (range >> s) < nb
    const int lg_nb = min(max(32 - __clz(n_el - 1), kLgMinBuckets), kLgMaxBuckets);
    const int nb = 1 << lg_nb;
    const int shift = range < (unsigned int)nb ? 0 : (31 - __clz((int)range)) - lg_nb + 1;
    if (!early_clear) {
      for (int i = tid; i <= nb; i += kPlanThreads) bucket[i] = 0;
      __syncthreads();
    }
    uint64_t mk[ITEMS];
    int mb[ITEMS], ms[ITEMS];
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) {
      const int g = tid + e * kPlanThreads;
      mk[e] = (g < n_keys) ? keys[g] : 0ull;
      mb[e] = 0;
      ms[e] = 0;
      if (mk[e]) {
        mb[e] = (int)((hi - (unsigned int)(mk[e] >> 32)) >> shift);
        ms[e] = atomicAdd(&bucket[mb[e]], 1);
      }
    }
    __syncthreads();
    // exclusive scan of the bucket counts (nb <= 4096: up to 4 per thread)
    const int per = (nb + kPlanThreads - 1) / kPlanThreads;
    int cnt_local = 0, big = 0;
    for (int q = 0; q < per; ++q) {
      const int i = tid * per + q;
      if (i < nb) {
        cnt_local += bucket[i];
        big = max(big, bucket[i]);
      }
    }
    if (big > kMaxBucketFill) atomicMax(&s_maxb, big);
    int total_cnt;
    // the barrier after the offsets below closes the scan
    int run = block_excl_scan_open<int, kPlanThreads>(cnt_local, w32, &total_cnt);
    for (int q = 0; q < per; ++q) {
      const int i = tid * per + q;
      if (i < nb) {
        const int c = bucket[i];
        bucket[i] = run;
        run += c;
      }
    }
    if (tid == 0) bucket[nb] = total_cnt;
    __syncthreads();
    if (s_maxb) {
      // a crowded bucket (many equal or nearly equal survivals): merge the
      // per-request runs instead, O(n log B) whatever the values
      sorted = merge_runs(keys, aux, n_keys, span);
    } else {
#pragma unroll
      for (int e = 0; e < ITEMS; ++e) {
        if (mk[e]) aux[bucket[mb[e]] + ms[e]] = mk[e];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < ITEMS; ++e) {
        if (mk[e]) {
          const int b0 = bucket[mb[e]], b1 = bucket[mb[e] + 1];
          int rank = 0;
          for (int j = b0; j < b1; ++j) rank += aux[j] > mk[e] ? 1 : 0;
          keys[b0 + rank] = mk[e];
        }
      }
      __syncthreads();
    }
  }

  // ---- 3. exact tau scan, ratio sweep, argmax
  uint64_t x[ITEMS];
  long long fxv[ITEMS];
  long long local = 0;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    const bool in = e < ipt && base_i + e < n_el;
    x[e] = in ? sorted[base_i + e] : 0ull;
    fxv[e] = in ? fx40(key_s(x[e])) : 0;
    local += fxv[e];
  }
  long long total_fx;
  // w64 is not written again: no closing barrier
  const long long offset = block_excl_scan_open<long long, kPlanThreads>(local, w64, &total_fx);
  const long long base = (long long)B * (1ll << 40) + forced;
  // every thread has read its sorted keys (the scan's barrier), so the key
  // buffer is free: start the per-request counts of verify_lens in it; the
  // argmax barrier below orders these stores before the counting
  int32_t* cnt = reinterpret_cast<int32_t*>(lds);
  for (int r = tid; r < B; r += kPlanThreads) cnt[r] = lmin;

  const int lo_b = min(max(a.b_lo, 0), n_el);
  const int hi_b = a.b_hi < 0 ? n_el : min(a.b_hi, n_el);
  const double t_fixed = __dadd_rn((double)a.bias, (double)alpha_b);

  double tau_v[ITEMS + 1], ratio_v[ITEMS + 1];
  double best_r = -1.0;
  int best_b = 0x7fffffff;
  int cost_bad = 0;
  long long run_fx = base + offset;
  // 1D mode: index of the last probe at or below the thread's first total M
  // (0 when every probe is above it); later budgets walk forward from it
  int pi = 0;
  if (sps_mode) {
    const int m_first = m0 + (tid == 0 ? 0 : base_i + 1);
    int lo = 0, hi = a.sps_len - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pm[mid] <= m_first) lo = mid;
      else hi = mid - 1;
    }
    pi = lo;
  }
  // slot 0 of thread 0 is b = 0; slot t >= 1 is b = base_i + t
#pragma unroll
  for (int t = 0; t <= ITEMS; ++t) {
    int b;
    if (t == 0) {
      b = (tid == 0) ? 0 : -1;
    } else {
      run_fx += fxv[t - 1];
      b = (t <= ipt && base_i + t <= n_el) ? base_i + t : -1;
    }
    tau_v[t] = 0.0;
    ratio_v[t] = 0.0;
    if (b < 0) continue;
    const long long tfx = (t == 0) ? base : run_fx;
    const double tau = __ll2double_rn(tfx) * 0x1p-40;
    double ratio;
    bool cost_ok;
    if (sps_mode) {
      const int M = m0 + b;
      while (pi + 1 < a.sps_len && s_pm[pi + 1] <= M) ++pi;
      const float S = s_ps[pi];
      ratio = __dmul_rn(tau, (double)S);
      cost_ok = S > 0.0f && S <= FLT_MAX;
    } else {
      const double T = __dadd_rn(t_fixed, (double)(t == 0 ? th0 : th[t - 1]));
      ratio = __ddiv_rn(tau, T);
      cost_ok = T > 0.0 && T <= DBL_MAX;
    }
    tau_v[t] = tau;
    ratio_v[t] = ratio;
    if (b >= lo_b && b <= hi_b) {
      if (!cost_ok) cost_bad = 1;
      else if (better(ratio, b, best_r, best_b)) {
        best_r = ratio;
        best_b = b;
      }
    }
  }
  if (cost_bad) atomicOr(&s_flags, DSPARK_DATA_BAD_COST);
  const int lane = lane_id(), wave = tid / kWave;
  {
    double wr;
    int wbst;
    lane_argmax<false>(best_r, best_b, ~0ull, wr, wbst);
    if (lane == 0) {
      wratio[wave] = wr;
      wb[wave] = wbst;
    }
  }
  __syncthreads();
  if (s_flags) {
    fallback<PACK>(a, p, s_flags, lds, w32, tier_lane, &pre);
    return;
  }
  // lane l of each 16-lane row holds wave l's pair; waves ascend in b
  double br;
  int bstar;
  lane_argmax<true>(wratio[lane & 15], wb[lane & 15], 0xFFFFull, br, bstar);

#pragma unroll
  for (int t = 0; t <= ITEMS; ++t) {
    const int b = (t == 0) ? (tid == 0 ? 0 : -1) : ((t <= ipt && base_i + t <= n_el) ? base_i + t : -1);
    if (b < 0) continue;
    if (a.sweep) {
      a.sweep[2 * b] = tau_v[t];
      a.sweep[2 * b + 1] = ratio_v[t];
    }
    if (b == bstar) {
      a.val[0] = tau_v[t];
      a.val[1] = ratio_v[t];
    }
  }
  if (a.sweep) {
    for (int b = n_el + 1 + tid; b < B * G + 1; b += kPlanThreads) {
      a.sweep[2 * b] = __builtin_nan("");
      a.sweep[2 * b + 1] = __builtin_nan("");
    }
  }

  // graph-tier alignment: fill the tier the chosen total already pays for
  int bexec = bstar;
  if (PACK && a.align) {
    const int total = m0 + bstar;
    const int tier = pick_tier(tier_lane, p.ntiers, total);
    bexec = min(bstar + (tier - total), n_el);
  }

  // ---- 4. verify_lens = L_min + #(first b_exec keys of each request)
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    if (e < ipt && base_i + e < bexec) atomicAdd(&cnt[key_r(x[e])], 1);
  }
  __syncthreads();
  for (int r = tid; r < B; r += kPlanThreads) a.lens[r] = cnt[r];
  if (tid == 0) {
    a.meta[0] = bstar;
    a.meta[1] = n_el;
    a.meta[2] = 0;
    a.meta[3] = m0 + bexec;
  }
  if (PACK) pack_block<kPlanThreads, kPackPrefetch>(p, cnt, cnt + B, w32, tier_lane, 0, &pre);
}

}  // namespace

size_t plan_lds_bytes(int B, int gamma, int n_keys) {
  const size_t main = (size_t)n_keys * sizeof(uint64_t) + plan_x_bytes(B, gamma, n_keys);
  const size_t pk = (size_t)(2 * B + 1) * sizeof(int32_t);  // lens + cu for the fused pack
  return main > pk ? main : pk;
}

namespace {

template <bool PACK>
void launch_plan_items(const PlanArgs& a, const PackArgs& p, size_t lds, hipStream_t s) {
  const int items = (a.B * a.gamma + kPlanThreads - 1) / kPlanThreads;  // <= kMaxItems
  if (items <= 1) {
    hipLaunchKernelGGL((plan_kernel<PACK, 1>), dim3(1), dim3(kPlanThreads), lds, s, a, p);
  } else if (items <= 2) {
    hipLaunchKernelGGL((plan_kernel<PACK, 2>), dim3(1), dim3(kPlanThreads), lds, s, a, p);
  } else if (items <= 4) {
    hipLaunchKernelGGL((plan_kernel<PACK, 4>), dim3(1), dim3(kPlanThreads), lds, s, a, p);
  } else {
    hipLaunchKernelGGL((plan_kernel<PACK, kMaxItems>), dim3(1), dim3(kPlanThreads), lds, s, a, p);
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, const PackArgs* p, hipStream_t s) {
  const size_t lds = plan_lds_bytes(a.B, a.gamma, a.B * (a.lmax - a.lmin));
  if (p) {
    launch_plan_items<true>(a, *p, lds, s);
  } else {
    PackArgs none{};
    launch_plan_items<false>(a, none, lds, s);
  }
  return hipGetLastError();
}

}  // namespace dspark
