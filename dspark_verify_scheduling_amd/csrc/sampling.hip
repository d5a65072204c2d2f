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
// maximum m gets integer weights, every float step one IEEE float32 operation:
//   c = K / T (K = 94548.4609375f, the float32 nearest to 2^16 log2 e),
//   u = (m - x) * c, j = nearest integer to u (ties to even), W = 0 unless
//   j < 2^21; else n = j >> 16, h = (j >> 8) & 255, r = j & 255,
//   Y = B[h] - (((B[h] - B[h+1]) * r + 128) >> 8),  W = (Y + (2^n >> 1)) >> n
// with B[i] the nearest integer to 2^31 * 2^(-i/256) (exp_tables.h), so
// W ~ 2^31 exp((x - m) / T) and p = W / Z, Z = sum W < 2^49. Every decision
// below is then an exact integer comparison, the same in any summation order:
//   accept draft d  iff  (w >> 8) * Wq[d] * Zp < 2^24 * Wp[d] * Zq
//   draw with word w from integer weights v (total S): the smallest i whose
//   running sum exceeds floor((w >> 8) * S / 2^24)
//   residual weights max(0, Wp * Zq - Wq * Zp); all zero -> draw from p.
// The residual is summed as Zq * sum(Wp) - Zp * sum(Wq) over the tokens where
// it is positive, so per element only a membership test and two 64-bit
// additions are needed.
//
// Work is indexed by slot, not by packed row: target slot (r, j) is row
// cu[r] + j of request r and draft slot (r, k) is draft row r * gamma + k, so
// every statistic is taken at the temperature of the request that reads it.
// Kernels:
//   samp_max_kernel: per (slot, chunk of up to 2048 16-byte vectors), the
//     maximum with its first index (NaN highest), for every slot read.
//   samp_z_kernel: per (slot, chunk) of a sampling request, the row maximum
//     from the chunk maxima, then the chunk's sum of W (a second read).
//   samp_decide_kernel: one wave per request: the chain tests, lane k on
//     draft k + 1, the first rejection by ballot, every output except the
//     drawn token; a draw job for sampling requests.
//   samp_draw_kernel: one workgroup per draw job: each wave sums the weights
//     of a contiguous sixteenth of the row; the sixteenth holding the
//     crossing point is split over all 1024 threads (a few elements each) and
//     scanned; the thread holding it walks its elements in order.
#include <float.h>

#include "common.h"
#include "exp_tables.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned __int128 u128;

constexpr float kLog2e16 = 94548.4609375f;  // float32 nearest to 2^16 log2(e)
constexpr unsigned int kJmax = 1u << 21;     // from here on the weight is 0
constexpr int kRedWaves = kSampThreads / kWave;

__device__ inline float temp_coef(float T) { return __fdiv_rn(kLog2e16, T); }

// The integer weight of x in a row with maximum m (x <= m); Bt is the table
// in LDS. Branch-free: out-of-range values read entry 0 and are masked.
__device__ inline unsigned int weight(float x, float m, float c, const unsigned int* Bt) {
  const float u = __fmul_rn(__fsub_rn(m, x), c);  // >= 0, or +inf
  const bool in = u < (float)kJmax;
  // adding 1.5 * 2^23 rounds u in [0, 2^22) to the nearest integer (ties to
  // even) and leaves it in the low mantissa bits
  const unsigned int j = __float_as_uint(__fadd_rn(in ? u : 0.0f, 12582912.0f)) & 0x3FFFFFu;
  const bool ok = in && j < kJmax;
  const unsigned int n = (j >> 16) & 31u, h = (j >> 8) & 255u, r = j & 255u;
  const unsigned int b0 = Bt[h], b1 = Bt[h + 1];
  const unsigned int d = (b0 - b1) & 0xFFFFFFu;  // < 2^23; the mask admits the 24-bit multiplier
  const unsigned int y = b0 - ((d * r + 128u) >> 8);
  const unsigned int w = (y + ((1u << n) >> 1)) >> n;
  return ok ? w : 0u;
}

__device__ inline void load_table(unsigned int* Bt) {
  for (int i = threadIdx.x; i < kExp2Len; i += blockDim.x) Bt[i] = kExp2B[i];
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

// A row is unusable for sampling when its maximum is NaN or +inf (a NaN
// anywhere ranks highest) or -inf (no finite element).
__device__ inline bool key_bad(unsigned int k) { return k >= 0xFF000000u || k == 0u; }

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

__device__ inline int best_index(unsigned long long b) {
  return (int)(0xFFFFFFFFu - (unsigned int)b);
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline bool is_sampling_temp(float T) { return T > 0.0f && T <= FLT_MAX; }

// What a slot is: its row, whether a request reads it, whether it needs the
// weight sum, and the temperature of the request.
struct Slot {
  const unsigned char* row;
  bool live, samp;
  float T;
};

__device__ inline Slot resolve_slot(const SampArgs& a, int slot) {
  Slot s{nullptr, false, false, 0.0f};
  const int G = a.gamma, nt = a.B * (G + 1);
  const bool target = slot < nt;
  const int r = target ? slot / (G + 1) : (slot - nt) / G;
  const int idx = target ? slot - r * (G + 1) : slot - nt - r * G;
  const int total_eff = min(max(a.cu[a.B], 0), a.max_rows);
  const int c0 = a.cu[r], len = a.cu[r + 1] - c0;
  const bool ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  s.T = a.temps[r];
  const bool samp = is_sampling_temp(s.T);
  if (!ok || !(samp || s.T == 0.0f)) return s;
  if (target) {
    s.live = idx < len;
    s.row = a.tgt + (size_t)(c0 + idx) * a.ld_t;
  } else {
    s.live = samp && idx < len - 1;
    s.row = a.drf + (size_t)(slot - nt) * a.ld_q;
  }
  s.samp = s.live && samp;
  return s;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_max_kernel(SampArgs a) {
  __shared__ unsigned long long s_red[kRedWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  if (blockIdx.x == 0 && tid == 0) {
    a.meta[0] = a.cu[a.B];
    a.meta[1] = 0;
  }
  const int slot = blockIdx.x / a.chunks, ch = blockIdx.x - slot * a.chunks;
  if (slot >= a.B * (2 * a.gamma + 1)) return;
  const Slot s = resolve_slot(a, slot);
  if (!s.live) return;
  const u32x4* rv = reinterpret_cast<const u32x4*>(s.row);
  const int v0 = ch * a.chunk_vecs, v1 = min(v0 + a.chunk_vecs, a.nvec);
  u32x4 d[kSampVecsPerThread];
#pragma unroll
  for (int i = 0; i < kSampVecsPerThread; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    d[i] = v < v1 ? __builtin_nontemporal_load(rv + v) : (u32x4){0, 0, 0, 0};
  }
  unsigned long long best = 0;
  if (ch == a.chunks - 1 && tid < a.tail) {
    const int i = a.nvec * kEpv + tid;
    best = pack_best(f32_key(__float_as_uint(elem<DT>(s.row, i))), i);
  }
#pragma unroll
  for (int i = 0; i < kSampVecsPerThread; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    if (v < v1) {
      float x[kEpv];
      widen<DT>(d[i], x);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) {
        const unsigned long long b = pack_best(f32_key(__float_as_uint(x[e])), v * kEpv + e);
        best = b > best ? b : best;
      }
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) s_red[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = 0;
    for (int w = 0; w < kRedWaves; ++w) b = s_red[w] > b ? s_red[w] : b;
    a.kpart[(size_t)slot * a.chunks + ch] = b;
  }
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_z_kernel(SampArgs a) {
  __shared__ unsigned int s_B[kExp2Len];
  __shared__ unsigned long long s_red[kRedWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int slot = blockIdx.x / a.chunks, ch = blockIdx.x - slot * a.chunks;
  if (slot >= a.B * (2 * a.gamma + 1)) return;
  const Slot s = resolve_slot(a, slot);
  if (!s.samp) return;
  const u32x4* rv = reinterpret_cast<const u32x4*>(s.row);
  const int v0 = ch * a.chunk_vecs, v1 = min(v0 + a.chunk_vecs, a.nvec);
  u32x4 d[kSampVecsPerThread];
#pragma unroll
  for (int i = 0; i < kSampVecsPerThread; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    d[i] = v < v1 ? __builtin_nontemporal_load(rv + v) : (u32x4){0, 0, 0, 0};
  }
  load_table(s_B);
  unsigned long long best = 0;
  const unsigned long long* kp = a.kpart + (size_t)slot * a.chunks;
  for (int c = 0; c < a.chunks; ++c) best = kp[c] > best ? kp[c] : best;
  const unsigned int key = (unsigned int)(best >> 32);
  __syncthreads();  // the table
  if (key_bad(key)) {
    if (tid == 0) a.zpart[(size_t)slot * a.chunks + ch] = 0;
    return;
  }
  const float m = key_value(key), c = temp_coef(s.T);
  unsigned long long z = 0;
  if (ch == a.chunks - 1 && tid < a.tail) z = weight(elem<DT>(s.row, a.nvec * kEpv + tid), m, c, s_B);
#pragma unroll
  for (int i = 0; i < kSampVecsPerThread; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    if (v < v1) {
      float x[kEpv];
      widen<DT>(d[i], x);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) z += weight(x[e], m, c, s_B);
    }
  }
  z = wave_sum_u64(z);
  if (lane == 0) s_red[wave] = z;
  __syncthreads();
  if (tid == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < kRedWaves; ++w) t += s_red[w];
    a.zpart[(size_t)slot * a.chunks + ch] = t;
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
  const size_t tslot = (size_t)r * (G + 1), dslot = (size_t)a.B * (G + 1) + (size_t)r * G;
  const int C = a.chunks;
  // merged maximum key and weight sum of a slot
  auto key_of = [&](size_t slot) {
    const unsigned long long* p = a.kpart + slot * C;
    unsigned long long b = 0;
    for (int c = 0; c < C; ++c) b = p[c] > b ? p[c] : b;
    return b;
  };
  auto z_of = [&](size_t slot) {
    const unsigned long long* p = a.zpart + slot * C;
    unsigned long long z = 0;
    for (int c = 0; c < C; ++c) z += p[c];
    return z;
  };
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
      b |= key_bad((unsigned int)(key_of(tslot + j) >> 32));
      if (j < len - 1) b |= key_bad((unsigned int)(key_of(dslot + j) >> 32));
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
      a.jobs[r].mode = 0;
    }
    for (int j = lane; j <= G; j += kWave) out[j] = -1;
    return;
  }
  // lane k tests draft k + 1 against target slot k and draft slot k
  bool pass = false;
  if (lane < len - 1) {
    if (greedy) {
      pass = dr == best_index(key_of(tslot + lane));
    } else if (dr >= 0 && dr < a.V) {
      const float cT = temp_coef(T);
      const float mp = key_value((unsigned int)(key_of(tslot + lane) >> 32));
      const float mq = key_value((unsigned int)(key_of(dslot + lane) >> 32));
      const float xp = elem<DT>(a.tgt + (size_t)(c0 + lane) * a.ld_t, dr);
      const float xq = elem<DT>(a.drf + ((size_t)r * G + lane) * a.ld_q, dr);
      const unsigned long long wp = weight(xp, mp, cT, kExp2B);
      const unsigned long long wq = weight(xq, mq, cT, kExp2B);
      const unsigned int u = a.ra[(size_t)r * G + lane] >> 8;
      // u * wq < 2^55 and wp * Zq < 2^80: both sides below 2^104
      const u128 lhs = (u128)((unsigned long long)u * wq) * z_of(tslot + lane);
      const u128 rhs = ((u128)wp * z_of(dslot + lane)) << 24;
      pass = lhs < rhs;
    }
  }
  const unsigned long long fails = __ballot(lane < len - 1 && !pass);
  const int c = fails ? __builtin_ctzll(fails) : len - 1;
  const int am_c = greedy ? best_index(key_of(tslot + c)) : 0;
  for (int j = lane; j <= G; j += kWave) {  // G + 1 can be 65 columns
    if (j != c || greedy) out[j] = j == c ? am_c : (j < G ? dr : -1);
  }
  if (lane == 0) {
    a.num_correct[r] = c;
    a.commit[r] = c + 1;
    if (a.new_seq) a.new_seq[r] = prefix + c + 1;
    SampJob jb;
    jb.mode = greedy ? 0 : (fails ? 2 : 1);
    jb.prow = c0 + c;
    jb.qrow = r * G + c;
    jb.word = greedy ? 0u : a.rs[(size_t)r * (G + 1) + c];
    jb.col = c;
    jb.pad = 0;
    jb.mp = greedy ? 0.0f : key_value((unsigned int)(key_of(tslot + c) >> 32));
    jb.zp = greedy ? 0ull : z_of(tslot + c);
    jb.mq = jb.mode == 2 ? key_value((unsigned int)(key_of(dslot + c) >> 32)) : 0.0f;
    jb.zq = jb.mode == 2 ? z_of(dslot + c) : 0ull;
    a.jobs[r] = jb;
    if (greedy) a.bonus[r] = am_c;
  }
}

// The draw: p (plain) or the residual max(0, p - q) of a pair. A token i is
// a member when its residual weight Wp * Zq - Wq * Zp is positive (plain: when
// Wp > 0); running sums (A, B) of Wp and Wq over members give the running
// residual weight Zq * A - Zp * B (plain: Zq = 1, Zp = 0, B = 0).
struct DrawCtx {
  const unsigned char* p;
  const unsigned char* q;
  float mp, mq, cT;
  unsigned long long zp, zq;  // 0 and 1 for a plain draw
  double zpd, zqd;
  bool resid;
};

struct Pair {
  unsigned long long a, b;
};

__device__ inline bool member(const DrawCtx& c, unsigned int wp, unsigned int wq) {
  if (wp == 0) return false;
  if (!c.resid) return true;
  // products below 2^81, rounded once in float64 (Zp, Zq < 2^49 are exact):
  // a margin of 2^-50 decides every case but near-equality exactly
  const double x = (double)wp * c.zqd, y = (double)wq * c.zpd;
  if (x > y * (1.0 + 0x1p-50)) return true;
  if (x < y * (1.0 - 0x1p-50)) return false;
  return (u128)wp * c.zq > (u128)wq * c.zp;
}

__device__ inline u128 run_value(const DrawCtx& c, Pair s) {
  return (u128)c.zq * s.a - (u128)c.zp * s.b;
}

template <dspark_dtype DT>
__device__ inline void add_elem(const DrawCtx& c, int i, const unsigned int* Bt, Pair& s) {
  const unsigned int wp = weight(elem<DT>(c.p, i), c.mp, c.cT, Bt);
  const unsigned int wq = c.resid ? weight(elem<DT>(c.q, i), c.mq, c.cT, Bt) : 0u;
  if (member(c, wp, wq)) {
    s.a += wp;
    s.b += wq;
  }
}

// One workgroup per request with a draw job.
template <dspark_dtype DT>
__global__ __launch_bounds__(kSampDrawThreads) void samp_draw_kernel(SampArgs a) {
  constexpr int kWaves = kSampDrawThreads / kWave;
  __shared__ unsigned int s_B[kExp2Len];
  __shared__ Pair s_wsum[kWaves];
  __shared__ unsigned long long s_scan[kWaves];
  __shared__ int s_ctl[2];  // residual flag; crossing wave
  __shared__ u128 s_t;      // threshold left at the start of the crossing wave
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = blockIdx.x;
  const SampJob job = a.jobs[r];
  if (job.mode == 0) return;
  load_table(s_B);
  if (tid == 0) s_ctl[0] = job.mode == 2;
  __syncthreads();
  DrawCtx c;
  c.p = a.tgt + (size_t)job.prow * a.ld_t;
  c.mp = job.mp;
  c.cT = temp_coef(a.temps[r]);
  c.q = job.mode == 2 ? a.drf + (size_t)job.qrow * a.ld_q : nullptr;
  c.mq = job.mq;
  // wave w covers whole vectors [w * per, (w + 1) * per); the last wave also
  // takes the tail elements
  const int nvec = a.nvec, V = a.V;
  const int per = (nvec + kWaves - 1) / kWaves;
  const int v0 = min(wave * per, nvec), v1 = min(v0 + per, nvec);
  const u32x4* pv = reinterpret_cast<const u32x4*>(c.p);
  const u32x4* qv = reinterpret_cast<const u32x4*>(c.q);
  for (;;) {
    c.resid = s_ctl[0] != 0;
    c.zp = c.resid ? job.zp : 0ull;
    c.zq = c.resid ? job.zq : 1ull;
    c.zpd = (double)c.zp;
    c.zqd = (double)c.zq;
    Pair s{0, 0};
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
      for (int e = 0; e < kEpv; ++e) {
        const unsigned int wp = weight(x[e], c.mp, c.cT, s_B);
        const unsigned int wq = c.resid ? weight(y[e], c.mq, c.cT, s_B) : 0u;
        if (member(c, wp, wq)) {
          s.a += wp;
          s.b += wq;
        }
      }
    }
    if (wave == kWaves - 1 && lane < a.tail) add_elem<DT>(c, nvec * kEpv + lane, s_B, s);
    s.a = wave_sum_u64(s.a);
    s.b = wave_sum_u64(s.b);
    if (lane == 0) s_wsum[wave] = s;
    __syncthreads();
    if (tid == 0) {
      Pair tot{0, 0};
      for (int w = 0; w < kWaves; ++w) {
        tot.a += s_wsum[w].a;
        tot.b += s_wsum[w].b;
      }
      const u128 S = run_value(c, tot);
      if (S == 0 && c.resid) {
        s_ctl[0] = 0;  // p == q at this resolution: draw from p
        s_ctl[1] = -1;
      } else {
        const u128 t = ((u128)(job.word >> 8) * S) >> 24;  // S < 2^98
        Pair run{0, 0};
        int w = 0;
        for (; w < kWaves - 1; ++w) {
          const Pair nx{run.a + s_wsum[w].a, run.b + s_wsum[w].b};
          if (run_value(c, nx) > t) break;
          run = nx;
        }
        s_ctl[1] = w;
        s_t = t - run_value(c, run);
      }
    }
    __syncthreads();
    if (s_ctl[1] >= 0) break;
  }
  // the crossing wave's elements [e0, e1), a contiguous run of `each` per thread
  const int ws = s_ctl[1];
  const int e0 = min(ws * per, nvec) * kEpv;
  const int e1 = ws == kWaves - 1 ? V : min(ws * per + per, nvec) * kEpv;
  const int each = (e1 - e0 + kSampDrawThreads - 1) / kSampDrawThreads;
  const int l0 = min(e0 + tid * each, e1), l1 = min(l0 + each, e1);
  Pair mine{0, 0};
  for (int i = l0; i < l1; ++i) add_elem<DT>(c, i, s_B, mine);
  unsigned long long tot_a, tot_b;
  const unsigned long long ea =
      block_excl_scan<unsigned long long, kSampDrawThreads>(mine.a, s_scan, &tot_a);
  const unsigned long long eb =
      block_excl_scan<unsigned long long, kSampDrawThreads>(mine.b, s_scan, &tot_b);
  const u128 t = s_t;
  const u128 before = run_value(c, Pair{ea, eb});
  const u128 after = run_value(c, Pair{ea + mine.a, eb + mine.b});
  // exactly one thread has before <= t < after
  if (!(before <= t && t < after)) return;
  Pair run{ea, eb};
  int tok = l1 - 1;
  for (int i = l0; i < l1; ++i) {
    add_elem<DT>(c, i, s_B, run);
    if (run_value(c, run) > t) {
      tok = i;
      break;
    }
  }
  a.bonus[r] = tok;
  a.out_tokens[(size_t)r * (a.gamma + 1) + job.col] = tok;
}

template <dspark_dtype DT>
hipError_t launch_dt(const SampArgs& a, hipStream_t s) {
  const long long units = (long long)a.B * (2 * a.gamma + 1) * a.chunks;
  hipLaunchKernelGGL(samp_max_kernel<DT>, dim3(units > 0 ? (unsigned)units : 1u),
                     dim3(kSampThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.B == 0) return e;
  hipLaunchKernelGGL(samp_z_kernel<DT>, dim3((unsigned)units), dim3(kSampThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(samp_decide_kernel<DT>, dim3(a.B), dim3(kWave), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(samp_draw_kernel<DT>, dim3(a.B), dim3(kSampDrawThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sampling(const SampArgs& a, dspark_dtype dt, hipStream_t s) {
  return dt == DSPARK_BF16 ? launch_dt<DSPARK_BF16>(a, s) : launch_dt<DSPARK_F32>(a, s);
}

}  // namespace dspark
