// Chain speculative-sampling accept over packed target logits.
//
// Method sources: "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit"
// (akiyangdev) §五 (AcceptSampling: speculative-sampling acceptance over the
// draft-side probabilities that actually proposed each draft and the target
// probabilities, yielding correct_len and the bonus); "DSpark 自适应 Verify
// 怎样分配候选预算" (akiyangdev) §二 (a draft drawn from q is accepted with
// probability min(1, p/q); mean acceptance sum min(p, q) = 1 - TV); "DSpark
// confidence-scheduled speculative decoding" (charlestar), "截短为什么不会改变
// 目标分布" (accept, reject and the residual resample follow the speculative
// algorithm; random numbers keep their meaning under compaction).
//
// Probabilities at fixed resolution. A row x at temperature T > 0 with
// maximum m gets integer weights
//   t = RN64(RN64(m - x) * RN64(65536 / T)),  j = nearest integer to t,
//   W = 0 if t or j >= 455 * 4096, else
//   W = (((E0[j >> 12] * E1[(j >> 6) & 63] + 2^22) >> 23) * E2[j & 63] + 2^22) >> 23
// with the tables of exp_tables.h (W ~ 2^40 exp((x - m) / T)), and p = W / Z,
// Z = sum W. Every decision below is then an exact integer comparison, the
// same in any summation order:
//   accept draft d  iff  (w >> 8) * Wq[d] * Zp < 2^24 * Wp[d] * Zq
//   draw with word w from integer weights v (total S): the smallest i whose
//   running sum exceeds floor((w >> 8) * S / 2^24)
//   residual weights max(0, Wp * Zq - Wq * Zp); all zero -> draw from p.
//
// Kernels:
//   samp_row_kernel: one 1024-thread workgroup per live row (target rows, and
//     the draft rows of sampling requests). The row stays in registers (16
//     16-byte vectors per thread; longer rows stream the rest twice): pass 1
//     takes the maximum and its first index, pass 2 sums W.
//   samp_decide_kernel: one wave per request: the chain tests, lane k on
//     draft k + 1, the first rejection by ballot, every output except the
//     drawn token; a draw job for sampling requests.
//   samp_draw_kernel: one workgroup per draw job: each wave sums the weights
//     of a contiguous sixteenth of the row; the wave holding the crossing
//     point splits its range over its lanes; the lane holding it walks its
//     elements in order.
#include <float.h>

#include "common.h"
#include "exp_tables.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned __int128 u128;

constexpr int kWaves = kSampThreads / kWave;
constexpr int kE0Len = 455;
constexpr int kJmax = kE0Len * 4096;

struct Tables {
  const unsigned long long* e0;
  const unsigned int* e1;
  const unsigned int* e2;
};

__device__ inline unsigned long long weight(float x, double m, double s, const Tables& tb) {
  const double t = __dmul_rn(__dsub_rn(m, (double)x), s);
  if (!(t < (double)kJmax)) return 0;  // also NaN
  const int j = (int)__builtin_rint(t);
  if (j >= kJmax) return 0;
  const unsigned long long P =
      (tb.e0[j >> 12] * (unsigned long long)tb.e1[(j >> 6) & 63] + (1ull << 22)) >> 23;
  return (P * tb.e2[j & 63] + (1ull << 22)) >> 23;
}

// 32-bit order key: larger value -> larger key, -0 == +0, +inf -> 0xFF000000,
// every NaN -> 0xFF000001, -inf -> 0.
__device__ inline unsigned int f32_key(unsigned int b) {
  const unsigned int m = (unsigned int)((int)b >> 31);
  const unsigned int x = b ^ (m | 0x80000000u);
  const unsigned int k = x - (m + 0x00800000u);
  return k < 0xFF000001u ? k : 0xFF000001u;
}

// The float of a non-NaN key (both zeros decode to +0).
__device__ inline float key_value(unsigned int k) {
  return __uint_as_float(k >= 0x7F800000u ? k - 0x7F800000u : ~(k + 0x007FFFFFu));
}

template <dspark_dtype DT>
__device__ inline float elem(const unsigned char* row, int i) {
  if constexpr (DT == DSPARK_BF16) {
    return __uint_as_float((unsigned int)reinterpret_cast<const unsigned short*>(row)[i] << 16);
  } else {
    return reinterpret_cast<const float*>(row)[i];
  }
}

template <dspark_dtype DT>
__device__ inline void widen(const u32x4& d, float* x) {
  if constexpr (DT == DSPARK_BF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned int v = d[w];
      x[2 * w] = __uint_as_float(v << 16);
      x[2 * w + 1] = __uint_as_float(v & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = __uint_as_float(d[w]);
  }
}

__device__ inline unsigned long long pack_best(unsigned int key, unsigned int idx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline u128 shfl_xor_u128(u128 v, int off) {
  const unsigned long long lo = __shfl_xor((unsigned long long)v, off, kWave);
  const unsigned long long hi = __shfl_xor((unsigned long long)(v >> 64), off, kWave);
  return ((u128)hi << 64) | lo;
}

__device__ inline u128 shfl_up_u128(u128 v, int off) {
  const unsigned long long lo = __shfl_up((unsigned long long)v, off, kWave);
  const unsigned long long hi = __shfl_up((unsigned long long)(v >> 64), off, kWave);
  return ((u128)hi << 64) | lo;
}

__device__ inline u128 wave_sum_u128(u128 v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += shfl_xor_u128(v, off);
  return v;
}

__device__ inline u128 wave_incl_scan_u128(u128 v) {
  const int lane = lane_id();
  for (int off = 1; off < kWave; off <<= 1) {
    const u128 o = shfl_up_u128(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// floor(c * S / 2^24) for c < 2^24 and S < 2^120, without overflow.
__device__ inline u128 draw_threshold(unsigned int c, u128 S) {
  const unsigned long long lo = (unsigned long long)S, hi = (unsigned long long)(S >> 64);
  return (((u128)c * hi) << 40) + (((u128)c * lo) >> 24);
}

__device__ inline double temp_scale(float T) { return __ddiv_rn(65536.0, (double)T); }

__device__ inline bool is_sampling_temp(float T) { return T > 0.0f && T <= FLT_MAX; }

// Request of packed row i: the last r with cu[r] <= i (any r in [0, B) when
// cu is malformed; such a request's stats are never used).
__device__ inline int row_request(const int32_t* cu, int B, int i) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_row_kernel(SampArgs a) {
  __shared__ unsigned long long s_e0[kE0Len];
  __shared__ unsigned int s_e1[64], s_e2[64];
  __shared__ unsigned long long s_red[kWaves];
  __shared__ int s_job[3];  // live, needs Z, request
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int job = blockIdx.x;
  if (job == 0 && tid == 0) {
    a.meta[0] = a.cu[a.B];
    a.meta[1] = 0;
  }
  if (tid == 0) {
    int live = 0, needz = 0, r = 0;
    if (job < a.max_rows) {
      const int total = a.cu[a.B];
      const int total_eff = min(max(total, 0), a.max_rows);
      if (job < total_eff) {
        live = 1;
        r = a.B > 0 ? row_request(a.cu, a.B, job) : 0;
        needz = a.B > 0 && is_sampling_temp(a.temps[r]);
      }
    } else if (job - a.max_rows < a.B * a.gamma) {
      const int q = job - a.max_rows;
      r = q / a.gamma;
      const int k = q - r * a.gamma + 1;
      const int len = a.cu[r + 1] - a.cu[r];
      live = needz = is_sampling_temp(a.temps[r]) && k <= len - 1 && len <= a.gamma + 1;
    }
    s_job[0] = live;
    s_job[1] = needz;
    s_job[2] = r;
  }
  for (int i = tid; i < kE0Len; i += kSampThreads) s_e0[i] = kExpE0[i];
  if (tid < 64) {
    s_e1[tid] = kExpE1[tid];
    s_e2[tid] = kExpE2[tid];
  }
  __syncthreads();
  if (!s_job[0]) return;
  const bool target = job < a.max_rows;
  const unsigned char* row = target ? a.tgt + (size_t)job * a.ld_t
                                    : a.drf + (size_t)(job - a.max_rows) * a.ld_q;
  const u32x4* rv = reinterpret_cast<const u32x4*>(row);
  const int nvec = a.nvec;
  u32x4 d[kSampRegSlots];
#pragma unroll
  for (int s = 0; s < kSampRegSlots; ++s) {
    const int v = s * kSampThreads + tid;
    d[s] = v < nvec ? __builtin_nontemporal_load(rv + v) : (u32x4){0, 0, 0, 0};
  }
  const int tail_i = nvec * kEpv + tid;
  const bool has_tail = tid < a.tail;
  const float xt = has_tail ? elem<DT>(row, tail_i) : 0.0f;
  // pass 1: maximum, first index, NaN highest
  unsigned long long best = has_tail ? pack_best(f32_key(__float_as_uint(xt)), tail_i) : 0;
#pragma unroll
  for (int s = 0; s < kSampRegSlots; ++s) {
    const int v = s * kSampThreads + tid;
    if (v < nvec) {
      float x[kEpv];
      widen<DT>(d[s], x);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) {
        const unsigned long long b = pack_best(f32_key(__float_as_uint(x[e])), v * kEpv + e);
        best = b > best ? b : best;
      }
    }
  }
  for (int v = kSampRegSlots * kSampThreads + tid; v < nvec; v += kSampThreads) {
    float x[kEpv];
    widen<DT>(rv[v], x);
#pragma unroll
    for (int e = 0; e < kEpv; ++e) {
      const unsigned long long b = pack_best(f32_key(__float_as_uint(x[e])), v * kEpv + e);
      best = b > best ? b : best;
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) s_red[wave] = best;
  __syncthreads();
  best = lane < kWaves ? s_red[lane] : 0;
  best = wave_max_u64(best);
  const unsigned int key = (unsigned int)(best >> 32);
  const int am = (int)(0xFFFFFFFFu - (unsigned int)best);
  const int bad = key >= 0xFF000000u || key == 0u;
  const float m = bad ? 0.0f : key_value(key);
  SampRowStat* st = target ? a.tstat + job : a.dstat + (job - a.max_rows);
  if (!s_job[1] || bad) {
    if (tid == 0) {
      st->Z = 0;
      st->m = m;
      st->am = am;
      st->bad = bad;
    }
    return;
  }
  // pass 2: the sum of the integer weights
  const Tables tb{s_e0, s_e1, s_e2};
  const double md = (double)m, sc = temp_scale(a.temps[s_job[2]]);
  unsigned long long z = has_tail ? weight(xt, md, sc, tb) : 0;
#pragma unroll
  for (int s = 0; s < kSampRegSlots; ++s) {
    const int v = s * kSampThreads + tid;
    if (v < nvec) {
      float x[kEpv];
      widen<DT>(d[s], x);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) z += weight(x[e], md, sc, tb);
    }
  }
  for (int v = kSampRegSlots * kSampThreads + tid; v < nvec; v += kSampThreads) {
    float x[kEpv];
    widen<DT>(rv[v], x);
#pragma unroll
    for (int e = 0; e < kEpv; ++e) z += weight(x[e], md, sc, tb);
  }
  __syncthreads();  // s_red is reused
  z = block_sum<unsigned long long, kSampThreads>(z, s_red);
  if (tid == 0) {
    st->Z = z;
    st->m = m;
    st->am = am;
    st->bad = 0;
  }
}

// One wave per request.
template <dspark_dtype DT>
__global__ __launch_bounds__(kWave) void samp_decide_kernel(SampArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x, G = a.gamma;
  const int total = a.cu[a.B];
  const int total_eff = min(max(total, 0), a.max_rows);
  const int c0 = a.cu[r];
  const int len = a.cu[r + 1] - c0;
  const float T = a.temps[r];
  const int prefix = a.prefix ? a.prefix[r] : 0;
  const int dr = lane < G ? a.drafts[(size_t)r * G + lane] : 0;
  int status = 0;
  const bool ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  const bool greedy = T == 0.0f;
  const bool samp = is_sampling_temp(T);
  if (!ok) {
    status = DSPARK_DATA_BAD_LENS;
  } else if (!greedy && !samp) {
    status = DSPARK_DATA_BAD_CONF;
  } else if (samp) {
    bool b = false;
    for (int j = lane; j < len; j += kWave) {  // len can be 65
      b |= a.tstat[c0 + j].bad != 0;
      if (j < len - 1) b |= a.dstat[(size_t)r * G + j].bad != 0;
    }
    if (__ballot(b)) status = DSPARK_DATA_BAD_LOGITS;
  }
  int32_t* out = a.out_tokens + (size_t)r * (G + 1);
  if (status) {
    if (lane == 0) {
      atomicOr(a.meta + 1, status);
      a.num_correct[r] = 0;
      a.bonus[r] = -1;
      a.commit[r] = 0;
      if (a.new_seq) a.new_seq[r] = prefix;
    }
    for (int j = lane; j <= G; j += kWave) out[j] = -1;
    if (lane == 0) a.jobs[r].mode = 0;
    return;
  }
  // lane k tests draft k + 1 against target row k and draft row k
  bool pass = false;
  if (lane < len - 1) {
    if (greedy) {
      pass = dr == a.tstat[c0 + lane].am;
    } else if (dr >= 0 && dr < a.V) {
      const Tables tb{kExpE0, kExpE1, kExpE2};
      const SampRowStat sp = a.tstat[c0 + lane];
      const SampRowStat sq = a.dstat[(size_t)r * G + lane];
      const double sc = temp_scale(T);
      const float xp = elem<DT>(a.tgt + (size_t)(c0 + lane) * a.ld_t, dr);
      const float xq = elem<DT>(a.drf + ((size_t)r * G + lane) * a.ld_q, dr);
      const unsigned long long wp = weight(xp, (double)sp.m, sc, tb);
      const unsigned long long wq = weight(xq, (double)sq.m, sc, tb);
      const unsigned int u = a.ra[(size_t)r * G + lane] >> 8;
      // u * wq < 2^64 and wp * Zq < 2^98: both sides below 2^122
      const u128 lhs = (u128)((unsigned long long)u * wq) * sp.Z;
      const u128 rhs = ((u128)wp * sq.Z) << 24;
      pass = lhs < rhs;
    }
  }
  const unsigned long long fails = __ballot(lane < len - 1 && !pass);
  const int c = fails ? __builtin_ctzll(fails) : len - 1;
  for (int j = lane; j <= G; j += kWave) {  // G + 1 can be 65 columns
    if (j != c || greedy) out[j] = j == c ? a.tstat[c0 + c].am : (j < G ? dr : -1);
  }
  if (lane == 0) {
    a.num_correct[r] = c;
    a.commit[r] = c + 1;
    if (a.new_seq) a.new_seq[r] = prefix + c + 1;
    SampJob j;
    j.mode = greedy ? 0 : (fails ? 2 : 1);
    j.prow = c0 + c;
    j.qrow = r * G + c;
    j.word = greedy ? 0u : a.rs[(size_t)r * (G + 1) + c];
    j.col = c;
    j.pad = 0;
    a.jobs[r] = j;
    if (greedy) a.bonus[r] = a.tstat[c0 + c].am;
  }
}

// Weight of element i of the draw: Wp, or max(0, Wp * Zq - Wq * Zp).
struct DrawCtx {
  const unsigned char* p;
  const unsigned char* q;
  double mp, mq, sc;
  unsigned long long zp, zq;
  bool resid;
};

__device__ inline u128 draw_weight(const DrawCtx& c, float xp, float xq, const Tables& tb) {
  const unsigned long long wp = weight(xp, c.mp, c.sc, tb);
  if (!c.resid) return wp;
  const unsigned long long wq = weight(xq, c.mq, c.sc, tb);
  const u128 a = (u128)wp * c.zq, b = (u128)wq * c.zp;
  return a > b ? a - b : 0;
}

template <dspark_dtype DT>
__device__ inline u128 draw_weight_at(const DrawCtx& c, int i, const Tables& tb) {
  return draw_weight(c, elem<DT>(c.p, i), c.resid ? elem<DT>(c.q, i) : 0.0f, tb);
}

// One workgroup per request with a draw job.
template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_draw_kernel(SampArgs a) {
  __shared__ unsigned long long s_e0[kE0Len];
  __shared__ unsigned int s_e1[64], s_e2[64];
  __shared__ u128 s_wsum[kWaves];
  __shared__ int s_ctl[2];  // residual flag; crossing wave
  __shared__ u128 s_t;      // threshold left inside the crossing wave
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = blockIdx.x;
  const SampJob job = a.jobs[r];
  if (job.mode == 0) return;
  for (int i = tid; i < kE0Len; i += kSampThreads) s_e0[i] = kExpE0[i];
  if (tid < 64) {
    s_e1[tid] = kExpE1[tid];
    s_e2[tid] = kExpE2[tid];
  }
  if (tid == 0) s_ctl[0] = job.mode == 2;
  __syncthreads();
  const Tables tb{s_e0, s_e1, s_e2};
  const SampRowStat sp = a.tstat[job.prow];
  DrawCtx c;
  c.p = a.tgt + (size_t)job.prow * a.ld_t;
  c.mp = (double)sp.m;
  c.zp = sp.Z;
  c.sc = temp_scale(a.temps[r]);
  if (job.mode == 2) {
    const SampRowStat sq = a.dstat[job.qrow];
    c.q = a.drf + (size_t)job.qrow * a.ld_q;
    c.mq = (double)sq.m;
    c.zq = sq.Z;
  } else {
    c.q = nullptr;
    c.mq = 0.0;
    c.zq = 0;
  }
  // wave w covers elements [w * per * kEpv, ...) in whole vectors; the last
  // wave also takes the tail
  const int nvec = a.nvec, V = a.V;
  const int per = (nvec + kWaves - 1) / kWaves;
  const int v0 = min(wave * per, nvec), v1 = min(v0 + per, nvec);
  const u32x4* pv = reinterpret_cast<const u32x4*>(c.p);
  const u32x4* qv = reinterpret_cast<const u32x4*>(c.q);
  for (;;) {
    c.resid = s_ctl[0] != 0;
    u128 sum = 0;
    for (int v = v0 + lane; v < v1; v += kWave) {
      float x[kEpv], y[kEpv];
      widen<DT>(__builtin_nontemporal_load(pv + v), x);
      if (c.resid) {
        widen<DT>(__builtin_nontemporal_load(qv + v), y);
      } else {
#pragma unroll
        for (int e = 0; e < kEpv; ++e) y[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < kEpv; ++e) sum += draw_weight(c, x[e], y[e], tb);
    }
    if (wave == kWaves - 1 && lane < a.tail) sum += draw_weight_at<DT>(c, nvec * kEpv + lane, tb);
    sum = wave_sum_u128(sum);
    if (lane == 0) s_wsum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
      u128 S = 0;
      for (int w = 0; w < kWaves; ++w) S += s_wsum[w];
      if (S == 0 && c.resid) {
        s_ctl[0] = 0;  // p == q at this resolution: draw from p
        s_ctl[1] = -1;
      } else {
        u128 t = draw_threshold(job.word >> 8, S), run = 0;
        int w = 0;
        while (w < kWaves - 1 && run + s_wsum[w] <= t) run += s_wsum[w++];
        s_ctl[1] = w;
        s_t = t - run;
      }
    }
    __syncthreads();
    if (s_ctl[1] >= 0) break;
  }
  const int ws = s_ctl[1];
  if (wave != ws) return;
  // the crossing wave: contiguous element ranges per lane
  const int e0 = min(ws * per, nvec) * kEpv;
  const int e1 = ws == kWaves - 1 ? V : min(ws * per + per, nvec) * kEpv;
  const int each = (e1 - e0 + kWave - 1) / kWave;
  const int l0 = min(e0 + lane * each, e1), l1 = min(l0 + each, e1);
  u128 mine = 0;
  for (int i = l0; i < l1; ++i) mine += draw_weight_at<DT>(c, i, tb);
  const u128 incl = wave_incl_scan_u128(mine);
  const u128 t = s_t;
  const unsigned long long cross = __ballot(incl > t);
  const int ls = cross ? __builtin_ctzll(cross) : kWave - 1;
  if (lane != ls) return;
  u128 run = incl - mine;
  int tok = l1 > l0 ? l1 - 1 : e1 - 1;
  for (int i = l0; i < l1; ++i) {
    run += draw_weight_at<DT>(c, i, tb);
    if (run > t) {
      tok = i;
      break;
    }
  }
  a.bonus[r] = tok;
  a.out_tokens[(size_t)r * (a.gamma + 1) + job.col] = tok;
}

}  // namespace

hipError_t launch_sampling(const SampArgs& a, dspark_dtype dt, hipStream_t s) {
  const int rows = a.max_rows + a.B * a.gamma;
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(samp_row_kernel<DSPARK_BF16>, dim3(rows > 0 ? rows : 1), dim3(kSampThreads),
                       0, s, a);
  } else {
    hipLaunchKernelGGL(samp_row_kernel<DSPARK_F32>, dim3(rows > 0 ? rows : 1), dim3(kSampThreads),
                       0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.B == 0) return e;
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(samp_decide_kernel<DSPARK_BF16>, dim3(a.B), dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL(samp_decide_kernel<DSPARK_F32>, dim3(a.B), dim3(kWave), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(samp_draw_kernel<DSPARK_BF16>, dim3(a.B), dim3(kSampThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(samp_draw_kernel<DSPARK_F32>, dim3(a.B), dim3(kSampThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
