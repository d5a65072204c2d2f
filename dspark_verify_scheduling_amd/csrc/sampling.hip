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
// Probabilities as integer weights. A row x at temperature T > 0 with
// maximum m gets, per element:
//   c = K / T (K = 94548.4609375f, the float32 nearest to 2^16 log2 e; the
//     temperature is in the domain while c is finite),
//   t = RN32((x - m) * (c * 2^-16) + 31), one fused multiply-add,
//   W = 2^t rounded to the nearest integer (ties to even), 2^t from the
//     hardware base-2 exponential (v_exp_f32, within 0.8 of a float32 unit
//     in the last place on gfx950),
// so W is 2^31 exp((x - m) / T) within a relative 4e-6 plus half a unit, the
// maximum's own weight is 2^31, and p = W / Z with Z = sum W <= V 2^31.
// Every decision below is then an exact integer comparison, the same in any
// summation order:
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
// Kernels (chunks are 2048 16-byte vectors, the last one partial):
//   samp_rowstat_kernel (rows of 1024 to 16384 vectors): the statistics of
//     every slot read with one read of its row: the maximum key (with its
//     first index for a greedy row), then the per-chunk sums of W.
//   Other rows take two kernels instead:
//   samp_max_kernel: per (slot, chunk), the maximum with its first index
//     (NaN highest), for every slot read.
//   samp_z_kernel: per (slot, chunk) of a sampling request, the row maximum
//     from the chunk maxima, then the chunk's sum of W (a second read).
//   samp_decide_kernel: one wave per request: the chain tests, lane k on
//     draft k + 1, the first rejection by ballot, every output except the
//     drawn token; a draw job for sampling requests.
//   samp_rsum_kernel: per (request, chunk, half chunk) of a residual draw,
//     the sums of Wp and Wq over the tokens where the residual is positive.
//   samp_draw_kernel: one workgroup per draw job: the crossing chunk from the
//     chunk sums (the weight sums for a plain draw), then that chunk split
//     over all 1024 threads (a few elements each) and scanned; the thread
//     holding the crossing point hands its elements to one wave, which scans
//     them one per lane.
#include <float.h>

#include <algorithm>

#include "argmax_unit.h"
#include "common.h"

#pragma clang fp contract(off)

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned __int128 u128;

constexpr float kLog2e16 = 94548.4609375f;  // float32 nearest to 2^16 log2(e)
constexpr int kRedWaves = kSampThreads / kWave;
static_assert(kSampThreads == kAccThreads && kSampVecsPerThread == kAccVecsPerThread,
              "the max kernel runs the greedy accept's unit argmax");

// c = K / T of the file header (a temperature is in the domain while it is
// finite).
__device__ inline float temp_coef(float T) { return __fdiv_rn(kLog2e16, T); }

// W of the file header for x in a row with maximum m (x <= m), c = K / T:
// t = RN32((x - m) * (c * 2^-16) + 31) in one fused multiply-add (c * 2^-16
// is exact), the hardware base-2 exponential of t (v_exp_f32), then the
// nearest integer (ties to even). x = -inf gives t = -inf and W = 0; the row
// maximum gives t = 31 and W = 2^31.
__device__ inline float weight_f(float x, float m, float c) {
  const float t = __fmaf_rn(__fsub_rn(x, m), __fmul_rn(c, 0x1p-16f), 31.0f);
  return __builtin_rintf(__builtin_amdgcn_exp2f(t));
}

// The same weight as an integer (the float above is integer-valued and at
// most 2^31, so the conversion is exact).
__device__ inline unsigned int weight(float x, float m, float c) {
  return __float2uint_rz(weight_f(x, m, c));
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

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// A sampling temperature: positive, finite, and with a finite scale K / T.
__device__ inline bool is_sampling_temp(float T) {
  return T > 0.0f && T <= FLT_MAX && temp_coef(T) <= FLT_MAX;
}

// What a slot is: its row, whether a request reads it, whether it needs the
// weight sum, and the temperature of the request.
struct Slot {
  const unsigned char* row;
  bool live, samp;
  float T;
};

// A slot's request r and its index in the request's target or draft slots.
struct SlotIdx {
  int r, idx;
  bool target;
};

__device__ inline SlotIdx slot_index(const SampArgs& a, int slot) {
  const int G = a.gamma, nt = a.B * (G + 1);
  SlotIdx x;
  x.target = slot < nt;
  x.r = x.target ? slot / (G + 1) : (slot - nt) / G;
  x.idx = x.target ? slot - x.r * (G + 1) : slot - nt - x.r * G;
  return x;
}

// Whether a request reads the slot, from its request's cu[r], cu[r + 1] and
// temperature (total_eff = the packed total clamped to [0, max_rows]).
__device__ inline bool slot_live(const SampArgs& a, const SlotIdx& x, int total_eff, int c0, int c1,
                                 float T) {
  const int G = a.gamma, len = c1 - c0;
  const bool ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  const bool samp = is_sampling_temp(T);
  if (!ok || !(samp || T == 0.0f)) return false;
  return x.target ? x.idx < len : samp && x.idx < len - 1;
}

__device__ inline Slot resolve_slot(const SampArgs& a, int slot) {
  Slot s{nullptr, false, false, 0.0f};
  const SlotIdx x = slot_index(a, slot);
  const int total_eff = min(max(a.cu[a.B], 0), a.max_rows);
  const int c0 = a.cu[x.r];
  s.T = a.temps[x.r];
  s.live = slot_live(a, x, total_eff, c0, a.cu[x.r + 1], s.T);
  if (!s.live) return s;
  s.row = x.target ? a.tgt + (size_t)(c0 + x.idx) * a.ld_t
                   : a.drf + (size_t)(slot - a.B * (a.gamma + 1)) * a.ld_q;
  s.samp = is_sampling_temp(s.T);
  return s;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_max_kernel(SampArgs a) {
  __shared__ argmax::UnitSmem sm;
  const int tid = threadIdx.x;
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
    // -0.0 fill: below any positive value, never a NaN
    d[i] = (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    if (v < v1) d[i] = __builtin_nontemporal_load(rv + v);
  }
  const unsigned long long best =
      argmax::unit_best<DT>(d, v0, v1, s.row, a.nvec, a.tail, ch == a.chunks - 1, sm);
  if (tid == 0) a.kpart[(size_t)slot * a.chunks + ch] = best;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_z_kernel(SampArgs a) {
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
  unsigned long long best = 0;
  const unsigned long long* kp = a.kpart + (size_t)slot * a.chunks;
#pragma unroll 8
  for (int c = 0; c < a.chunks; ++c) best = kp[c] > best ? kp[c] : best;
  if (argmax::best_bad<DT>(best)) {
    if (tid == 0) a.zpart[(size_t)slot * a.chunks + ch] = 0;
    return;
  }
  const float m = argmax::best_value<DT>(best), c = temp_coef(s.T);
  unsigned long long z = 0;
  if (ch == a.chunks - 1 && tid < a.tail) z = weight(elem<DT>(s.row, a.nvec * kEpv + tid), m, c);
#pragma unroll
  for (int i = 0; i < kSampVecsPerThread; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    if (v < v1) {
      float x[kEpv];
      widen<DT>(d[i], x);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) z += weight(x[e], m, c);
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

// Row statistics of the sampling slots with one read of each row: the
// maximum key, then the weight sums per chunk. One persistent 1024-thread
// workgroup per CU takes the live slots of rank blockIdx.x, blockIdx.x +
// gridDim.x, ... (ranks in slot order). A row stays in registers
// between the two passes: vector v in register slot v / 1024 of thread
// v % 1024, so slots 2c and 2c + 1 hold chunk c (chunks are 2048 vectors).
// While the weight pass consumes a register slot it reloads it with the
// workgroup's next row, so the next row streams in under this row's
// arithmetic; the maximum pass then takes the slots in the order they arrive.
// A greedy row gets the lowest index of its maximum instead of weight sums.
// Rows of 1024 to SLOTS * 1024 vectors; it also initializes accept_meta.
template <dspark_dtype DT, int SLOTS>
__global__ __launch_bounds__(kRsThreads) void samp_rowstat_kernel(SampArgs a) {
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  constexpr int kWaves = kRsThreads / kWave;
  constexpr int kChunks = (SLOTS + 1) / 2;
  __shared__ int s_list[kRsMaxList];
  __shared__ int s_scan[kWaves];
  __shared__ unsigned int s_key[kWaves];
  __shared__ unsigned int s_idx[kWaves];  // apart from s_key: waves may still read the key
  __shared__ int s_flag[kWaves];
  // per-thread chunk sums of the weight pass: [chunk][thread]
  __shared__ unsigned long long s_zl[kChunks][kRsThreads];
  // the wave index as a scalar: the per-wave LDS addresses need no registers
  const int tid = threadIdx.x, lane = lane_id(),
            wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nvec = a.nvec;

  if (blockIdx.x == 0 && tid == 0) {
    a.meta[0] = a.cu[a.B];
    a.meta[1] = 0;
  }
  // ---- this workgroup's rows: thread t looks at slots [t k, t k + k)
  // (k <= 64, which the host ensures), eight at a time so that a group's
  // loads are all in flight together, and keeps their liveness as bits
  const int nslots = a.B * (2 * a.gamma + 1);
  const int per = (nslots + kRsThreads - 1) / kRsThreads;
  const int s0 = tid * per;
  const int total_eff = min(max(a.cu[a.B], 0), a.max_rows);
  unsigned long long live = 0;
  for (int j0 = 0; j0 < per; j0 += 8) {
    SlotIdx x[8];
    int c0[8], c1[8];
    float T[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // loads at in-range indices, all issued first
      x[j] = slot_index(a, min(s0 + j0 + j, nslots - 1));
      c0[j] = a.cu[x[j].r];
      c1[j] = a.cu[x[j].r + 1];
      T[j] = a.temps[x[j].r];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = j0 + j;
      if (k < per && s0 + k < nslots && slot_live(a, x[j], total_eff, c0[j], c1[j], T[j]))
        live |= 1ull << k;
    }
  }
  int total = 0;
  int rank = block_excl_scan<int, kRsThreads>(__popcll(live), s_scan, &total);
  for (unsigned long long m = live; m; m &= m - 1, ++rank) {
    if (rank % (int)gridDim.x == (int)blockIdx.x) {
      const int i = rank / (int)gridDim.x;
      if (i < kRsMaxList) s_list[i] = s0 + __builtin_ctzll(m);
    }
  }
  __syncthreads();
  const int mine = total > (int)blockIdx.x ? (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
  const int n_rows = mine < kRsMaxList ? mine : kRsMaxList;  // the host sizes the grid for this
  if (n_rows == 0) return;

  // ---- prologue: the first row's register slots, unconditionally and in
  // order (an index past the row end reads its last vector, never used)
  Slot cur = resolve_slot(a, s_list[0]);
  const u32x4* rv = reinterpret_cast<const u32x4*>(cur.row);
  // a row's tail elements (after its last whole vector), one per lane <
  // tail, are loaded before its register slots, so that waiting for them
  // never waits for the slots; every lane loads (an index past the row end
  // reads its last element) and lanes >= tail use -inf instead
  const int ti = min(nvec * kEpv + tid, a.V - 1);
  float xr = elem<DT>(cur.row, ti);
  u32x4 r[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int v = i * kRsThreads + tid;
    r[i] = rv[v < nvec ? v : nvec - 1];
    __builtin_amdgcn_sched_barrier(0);
  }
  const u32x4 fill = DT == DSPARK_BF16 ? (u32x4){0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}
                                       : (u32x4){0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u};
  const int last_chunk = (nvec - 1) / kSampChunkVecs;

  for (int k = 0; k < n_rows; ++k) {
    // the row length through an opaque copy, so that the per-slot bounds
    // are formed where they are used rather than kept live across the loop
    int nvk = nvec;
    asm volatile("" : "+s"(nvk));
    const int slot = s_list[k];
    const float xt = tid < a.tail ? xr : -INFINITY;

    // ---- pass 1: the maximum key, slots in arrival order. The first use of
    // the row's last, partial slot stores it back with -inf in the lanes past
    // the row end (no maximum, zero weight); later uses read r[i] as it is.
    auto slot_vec = [&](int i) -> u32x4 {
      if ((i + 1) * kRsThreads > nvk) r[i] = i * kRsThreads + tid < nvk ? r[i] : fill;
      return r[i];
    };
    unsigned int key;
    if constexpr (DT == DSPARK_BF16) {
      // fast path: raw signed-16 maximum (exact for a positive maximum) and
      // NaN detection; the raw order is reversed for negatives
      argmax::i16x2 mi = (argmax::i16x2){(short)0xFF80, (short)0xFF80};
      argmax::u16x2 mu = (argmax::u16x2){0, 0};
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (i * kRsThreads < nvk) {
          const u32x4 d = slot_vec(i);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            mi = __builtin_elementwise_max(mi, argmax::as_i16x2(d[w]));
            mu = __builtin_elementwise_max(mu, argmax::as_u16x2(d[w]));
          }
        }
      }
      const unsigned int xt_w = (__float_as_uint(xt) >> 16) | 0xFF800000u;  // tail in the low half
      mi = __builtin_elementwise_max(mi, argmax::as_i16x2(xt_w));
      mu = __builtin_elementwise_max(mu, argmax::as_u16x2(xt_w));
      const int lm = max((int)mi[0], (int)mi[1]);
      const int lu = max((int)mu[0], (int)mu[1]);
      int v = (lm > 0x7F80 || lu > 0xFF80) ? 0x7FFFFFFF : lm;
      v = argmax::wave_max(v);
      if (lane == 0) s_flag[wave] = v;
      __syncthreads();
      int M = s_flag[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = max(M, s_flag[w]);
      if (M > 0 && M <= 0x7F80) {
        key = (unsigned int)M + 0x7F80u;
      } else {  // a non-positive maximum or a NaN: exact 16-bit keys
        unsigned int kk = 0;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
          if (i * kRsThreads < nvk) {
            const u32x4 d = r[i];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const unsigned int kw = argmax::bf16x2_keys(d[w]);
              kk = max(kk, max(kw & 0xFFFFu, kw >> 16));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (tid < a.tail) kk = max(kk, argmax::bf16x2_keys(__float_as_uint(xt) >> 16) & 0xFFFFu);
        kk = argmax::wave_max(kk);
        if (lane == 0) s_key[wave] = kk;
        __syncthreads();
        key = s_key[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) key = max(key, s_key[w]);
      }
    } else {
      unsigned int kk = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        if (i * kRsThreads < nvk) {
          const u32x4 d = slot_vec(i);
#pragma unroll
          for (int w = 0; w < 4; ++w) kk = max(kk, argmax::f32_key(d[w]));
        }
      }
      if (tid < a.tail) kk = max(kk, argmax::f32_key(__float_as_uint(xt)));
      kk = argmax::wave_max(kk);
      if (lane == 0) s_key[wave] = kk;
      __syncthreads();
      key = s_key[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) key = max(key, s_key[w]);
    }
    // a greedy row also needs the lowest index holding the maximum key (a
    // sampling row only the value: its index field is left 0)
    unsigned int idx = 0;
    if (!cur.samp) {
      unsigned int cand = 0xFFFFFFFFu;
      // element e of dword w of slot i: index (i * 1024 + tid) * kEpv + e;
      // walked from the end so that the last match kept is the first one
      if (tid < a.tail) {
        const unsigned int kt = DT == DSPARK_BF16
                                    ? (argmax::bf16x2_keys(__float_as_uint(xt) >> 16) & 0xFFFFu)
                                    : argmax::f32_key(__float_as_uint(xt));
        if (kt == key) cand = (unsigned int)(nvk * kEpv + tid);
      }
#pragma unroll
      for (int i = SLOTS - 1; i >= 0; --i) {
        if (i * kRsThreads < nvk) {
          const u32x4 d = r[i];
          const unsigned int base = (unsigned int)(i * kRsThreads + tid) * kEpv;
#pragma unroll
          for (int w = 3; w >= 0; --w) {
            if constexpr (DT == DSPARK_BF16) {
              const unsigned int kw = argmax::bf16x2_keys(d[w]);
              if ((kw >> 16) == key) cand = base + 2u * w + 1u;
              if ((kw & 0xFFFFu) == key) cand = base + 2u * w;
            } else {
              if (argmax::f32_key(d[w]) == key) cand = base + w;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      cand = argmax::wave_min(cand);
      if (lane == 0) s_idx[wave] = cand;
      __syncthreads();
      idx = s_idx[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) idx = min(idx, s_idx[w]);
    }
    const unsigned long long best = argmax::pack_best(key, idx);
    const bool bad = argmax::best_bad<DT>(best);
    const float m = argmax::best_value<DT>(best), c = temp_coef(cur.T);

    // ---- pass 2: weight sums per chunk, each register slot reloaded with
    // the next row once consumed (after the last row: the first 64 vectors of
    // the current row, the same 1 KB for every slot, unused)
    const bool more = k + 1 < n_rows;
    Slot nxt = cur;
    if (more) nxt = resolve_slot(a, s_list[k + 1]);
    const u32x4* nv = reinterpret_cast<const u32x4*>(nxt.row);
    const float xr_next = elem<DT>(nxt.row, ti);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) asm volatile("" : "+v"(r[i]));
    unsigned long long zc = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      if (cur.samp && !bad && i * kRsThreads < nvec) {
        const u32x4 d = r[i];
        float x[kEpv];
        widen<DT>(d, x);
#pragma unroll
        for (int e = 0; e < kEpv; ++e) zc += weight(x[e], m, c);
      }
      // both slots of a chunk are summed before either is reloaded (the
      // reload's address depends on an opaque copy of the thread index tied
      // to the sum, so the slots' words are consumed before it is issued)
      if (!(i & 1) && i != SLOTS - 1) continue;
#pragma unroll
      for (int i2 = (i & ~1); i2 <= i; ++i2) {
        int lt = tid;
        asm volatile("" : "+v"(lt), "+v"(zc));
        const int v = more ? i2 * kRsThreads + lt : (lt & (kWave - 1));
        r[i2] = nv[v < nvec ? v : nvec - 1];
      }
      if ((i & 1) || i == SLOTS - 1) {
        const int ch = i >> 1;
        if (ch == last_chunk && cur.samp && !bad && tid < a.tail) zc += weight(xt, m, c);
        s_zl[ch][tid] = zc;
        zc = 0;
      }
    }
    // wave w < chunks adds up chunk w's 1024 thread sums and stores the
    // chunk's partials; the next row writes s_zl only after its pass-1
    // barrier, which every wave reaches after these reads
    __syncthreads();
    if (wave < a.chunks) {
      unsigned long long t = 0;
      if (wave < kChunks) {
#pragma unroll
        for (int j = 0; j < kWaves; ++j) t += s_zl[wave][j * kWave + lane];
        t = wave_sum_u64(t);
      }
      if (lane == 0) {
        a.zpart[(size_t)slot * a.chunks + wave] = bad || !cur.samp ? 0ull : t;
        a.kpart[(size_t)slot * a.chunks + wave] = wave == 0 ? best : 0ull;
      }
    }
    cur = nxt;
    xr = xr_next;
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
#pragma unroll 8
    for (int c = 0; c < C; ++c) b = p[c] > b ? p[c] : b;
    return b;
  };
  auto z_of = [&](size_t slot) {  // the 65th row only
    const unsigned long long* p = a.zpart + slot * C;
    unsigned long long z = 0;
    for (int c = 0; c < C; ++c) z += p[c];
    return z;
  };
  int status = 0;
  const bool ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  const bool greedy = T == 0.0f;
  const bool samp = is_sampling_temp(T);
  // this lane's target slot and draft slot, merged once: the four partial
  // runs are read together, eight chunks a round, at slot indices clamped to
  // the request's own slots and chunk indices clamped to the last (a repeated
  // key leaves the maximum; a repeated sum term is not added); what a lane
  // does not own is dropped afterwards
  const bool mine_t = ok && (greedy || samp) && lane < len;
  const bool mine_d = ok && samp && lane < len - 1;
  unsigned long long kt = 0, kd = 0, zt = 0, zd = 0;
  {
    const size_t ts = (tslot + min(lane, G)) * C, ds = (dslot + min(lane, G - 1)) * C;
    for (int c0 = 0; c0 < C; c0 += 8) {
      unsigned long long v[4][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = min(c0 + e, C - 1);
        v[0][e] = a.kpart[ts + c];
        v[1][e] = a.kpart[ds + c];
        v[2][e] = a.zpart[ts + c];
        v[3][e] = a.zpart[ds + c];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kt = v[0][e] > kt ? v[0][e] : kt;
        kd = v[1][e] > kd ? v[1][e] : kd;
        zt += c0 + e < C ? v[2][e] : 0ull;
        zd += c0 + e < C ? v[3][e] : 0ull;
      }
    }
  }
  kt = mine_t ? kt : 0;
  kd = mine_d ? kd : 0;
  zt = mine_t && samp ? zt : 0;
  zd = mine_d ? zd : 0;
  if (!ok) {
    status = DSPARK_DATA_BAD_LENS;
  } else if (!greedy && !samp) {
    status = DSPARK_DATA_BAD_CONF;
  } else if (samp) {
    bool b = (mine_t && argmax::best_bad<DT>(kt)) || (mine_d && argmax::best_bad<DT>(kd));
    if (len > kWave) b |= argmax::best_bad<DT>(key_of(tslot + kWave));  // the 65th row
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
      pass = dr == argmax::best_index(kt);
    } else if (dr >= 0 && dr < a.V) {
      const float cT = temp_coef(T);
      const float mp = argmax::best_value<DT>(kt);
      const float mq = argmax::best_value<DT>(kd);
      const float xp = elem<DT>(a.tgt + (size_t)(c0 + lane) * a.ld_t, dr);
      const float xq = elem<DT>(a.drf + ((size_t)r * G + lane) * a.ld_q, dr);
      const unsigned long long wp = weight(xp, mp, cT);
      const unsigned long long wq = weight(xq, mq, cT);
      const unsigned int u = a.ra[(size_t)r * G + lane] >> 8;
      // u * wq < 2^55 and wp * Zq < 2^80: both sides below 2^104
      const u128 lhs = (u128)((unsigned long long)u * wq) * zt;
      const u128 rhs = ((u128)wp * zd) << 24;
      pass = lhs < rhs;
    }
  }
  const unsigned long long fails = __ballot(lane < len - 1 && !pass);
  const int c = fails ? __builtin_ctzll(fails) : len - 1;
  // the slot values of lane c (c <= len - 1 <= 64; slot 64 is merged directly)
  const unsigned long long kt_c = c < kWave ? __shfl(kt, c, kWave) : key_of(tslot + c);
  const unsigned long long kd_c = __shfl(kd, c < kWave ? c : 0, kWave);
  const unsigned long long zt_c = c < kWave ? __shfl(zt, c, kWave) : z_of(tslot + c);
  const unsigned long long zd_c = __shfl(zd, c < kWave ? c : 0, kWave);
  const int am_c = greedy ? argmax::best_index(kt_c) : 0;
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
    jb.mp = greedy ? 0.0f : argmax::best_value<DT>(kt_c);
    jb.zp = greedy ? 0ull : zt_c;
    jb.mq = jb.mode == 2 ? argmax::best_value<DT>(kd_c) : 0.0f;
    jb.zq = jb.mode == 2 ? zd_c : 0ull;
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
  float zpf, zqf;             // the same, rounded to float32
  bool resid;
};

struct Pair {
  unsigned long long a, b;
};

__device__ inline bool member(const DrawCtx& c, unsigned int wp, unsigned int wq) {
  if (wp == 0) return false;
  if (!c.resid) return true;
  // Wp Zq against Wq Zp (below 2^80) screened in float32: each side is within
  // 3 * 2^-24 relative of its exact value (three roundings), the margin
  // product within 2^-24, so a margin of 2^-20 decides every case it passes
  // correctly; near-equality is decided exactly
  const float x = (float)wp * c.zqf, y = (float)wq * c.zpf;
  if (x > y * (1.0f + 0x1p-20f)) return true;
  if (x < y * (1.0f - 0x1p-20f)) return false;
  return (u128)wp * c.zq > (u128)wq * c.zp;
}

__device__ inline u128 run_value(const DrawCtx& c, Pair s) {
  return (u128)c.zq * s.a - (u128)c.zp * s.b;
}

template <dspark_dtype DT>
__device__ inline void add_elem(const DrawCtx& c, int i, Pair& s) {
  const unsigned int wp = weight(elem<DT>(c.p, i), c.mp, c.cT);
  const unsigned int wq = c.resid ? weight(elem<DT>(c.q, i), c.mq, c.cT) : 0u;
  if (member(c, wp, wq)) {
    s.a += wp;
    s.b += wq;
  }
}

// member() summed over the valid vectors of dp (p) and dq (q) without
// branches: the float32 screen decides every element it can, and the few near
// equality (flagged) are decided exactly afterwards, in a second walk that
// only a wave holding one takes. A plain draw (not c.resid) sums Wp alone.
template <dspark_dtype DT, int N>
__device__ inline Pair member_sums(const DrawCtx& c, const u32x4 (&dp)[N], const u32x4 (&dq)[N],
                                   const bool (&valid)[N]) {
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  Pair s{0, 0};
  if (!c.resid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (valid[i]) {
        float x[kEpv];
        widen<DT>(dp[i], x);
#pragma unroll
        for (int e = 0; e < kEpv; ++e) s.a += weight(x[e], c.mp, c.cT);
      }
    }
    return s;
  }
  bool near = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (valid[i]) {
      float x[kEpv], y[kEpv];
      widen<DT>(dp[i], x);
      widen<DT>(dq[i], y);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) {
        const float fp = weight_f(x[e], c.mp, c.cT), fq = weight_f(y[e], c.mq, c.cT);
        const float xs = fp * c.zqf, ys = fq * c.zpf;
        const bool hi = xs > ys * (1.0f + 0x1p-20f), lo = xs < ys * (1.0f - 0x1p-20f);
        s.a += hi ? __float2uint_rz(fp) : 0u;
        s.b += hi ? __float2uint_rz(fq) : 0u;
        near |= !hi && !lo && fp != 0.0f;
      }
    }
  }
  if (__ballot(near)) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (near && valid[i]) {
        float x[kEpv], y[kEpv];
        widen<DT>(dp[i], x);
        widen<DT>(dq[i], y);
        for (int e = 0; e < kEpv; ++e) {
          const float fp = weight_f(x[e], c.mp, c.cT), fq = weight_f(y[e], c.mq, c.cT);
          const float xs = fp * c.zqf, ys = fq * c.zpf;
          const bool hi = xs > ys * (1.0f + 0x1p-20f), lo = xs < ys * (1.0f - 0x1p-20f);
          const unsigned int wp = __float2uint_rz(fp), wq = __float2uint_rz(fq);
          if (!hi && !lo && wp != 0 && member(c, wp, wq)) {
            s.a += wp;
            s.b += wq;
          }
        }
      }
    }
  }
  return s;
}

__device__ inline void set_mode(DrawCtx& c, const SampJob& job, bool resid) {
  c.resid = resid;
  c.zp = resid ? job.zp : 0ull;
  c.zq = resid ? job.zq : 1ull;
  c.zpf = (float)c.zp;
  c.zqf = (float)c.zq;
}

__device__ inline DrawCtx draw_ctx(const SampArgs& a, const SampJob& job, int r) {
  DrawCtx c;
  c.p = a.tgt + (size_t)job.prow * a.ld_t;
  c.mp = job.mp;
  c.cT = temp_coef(a.temps[r]);
  c.q = job.mode == 2 ? a.drf + (size_t)job.qrow * a.ld_q : nullptr;
  c.mq = job.mq;
  set_mode(c, job, job.mode == 2);
  return c;
}

// Per (request, chunk, part) of a residual draw: the member sums of Wp and
// Wq over part `part` of the chunk (kRsumParts equal parts; smaller
// workgroups keep more of them on a CU, loading while others sum).
constexpr int kRsumVecs = kSampVecsPerThread / kRsumParts;  // per thread
static_assert(kRsumVecs * kRsumParts == kSampVecsPerThread, "parts split a chunk evenly");

template <dspark_dtype DT>
__global__ __launch_bounds__(kSampThreads) void samp_rsum_kernel(SampArgs a) {
  __shared__ Pair s_red[kRedWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int part = blockIdx.x % kRsumParts, u = blockIdx.x / kRsumParts;
  const int r = u / a.chunks, ch = u - r * a.chunks;
  const SampJob job = a.jobs[r];
  if (job.mode != 2) return;
  const DrawCtx c = draw_ctx(a, job, r);
  const u32x4* pv = reinterpret_cast<const u32x4*>(c.p);
  const u32x4* qv = reinterpret_cast<const u32x4*>(c.q);
  const int v0 = ch * a.chunk_vecs + part * (kRsumVecs * kSampThreads);
  const int v1 = min(v0 + kRsumVecs * kSampThreads, min(ch * a.chunk_vecs + a.chunk_vecs, a.nvec));
  u32x4 dp[kRsumVecs], dq[kRsumVecs];
#pragma unroll
  for (int i = 0; i < kRsumVecs; ++i) {
    const int v = v0 + i * kSampThreads + tid;
    dp[i] = v < v1 ? __builtin_nontemporal_load(pv + v) : (u32x4){0, 0, 0, 0};
    dq[i] = v < v1 ? __builtin_nontemporal_load(qv + v) : (u32x4){0, 0, 0, 0};
  }
  bool valid[kRsumVecs];
#pragma unroll
  for (int i = 0; i < kRsumVecs; ++i) valid[i] = v0 + i * kSampThreads + tid < v1;
  Pair s = member_sums<DT, kRsumVecs>(c, dp, dq, valid);
  if (part == 0 && ch == a.chunks - 1 && tid < a.tail) add_elem<DT>(c, a.nvec * kEpv + tid, s);
  s.a = wave_sum_u64(s.a);
  s.b = wave_sum_u64(s.b);
  if (lane == 0) s_red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    Pair t{0, 0};
    for (int w = 0; w < kRedWaves; ++w) {
      t.a += s_red[w].a;
      t.b += s_red[w].b;
    }
    a.rpart[((size_t)u * kRsumParts + part) * 2] = t.a;
    a.rpart[((size_t)u * kRsumParts + part) * 2 + 1] = t.b;
  }
}

// One workgroup per request with a draw job: the crossing chunk from the
// per-chunk sums (residual: samp_rsum_kernel's halves added; plain: the
// weight sums of the target slot), then the chunk's elements split over the
// threads and scanned, then the crossing thread's elements one per lane of
// wave 0.
template <dspark_dtype DT>
__global__ __launch_bounds__(kSampDrawThreads) void samp_draw_kernel(SampArgs a) {
  constexpr int kWaves = kSampDrawThreads / kWave;
  __shared__ unsigned long long s_scan[kWaves], s_scan_b[kWaves];
  __shared__ int s_ctl[2];  // residual flag; crossing chunk
  __shared__ u128 s_t;      // threshold left at the start of the crossing chunk
  __shared__ Pair s_rs[kSampMaxChunks];            // residual chunk sums
  __shared__ unsigned long long s_zs[kSampMaxChunks];  // plain chunk sums
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int tid = threadIdx.x;
  const int r = blockIdx.x, C = a.chunks;
  const SampJob job = a.jobs[r];
  if (job.mode == 0) return;
  DrawCtx c = draw_ctx(a, job, r);
  if (tid < C) {  // one load per thread, not a chain of them in one thread
    s_zs[tid] = a.zpart[((size_t)r * (a.gamma + 1) + job.col) * C + tid];
    if (job.mode == 2) {  // the chunk's parts added up
      const unsigned long long* rp = a.rpart + ((size_t)r * C + tid) * kRsumParts * 2;
      Pair t{0, 0};
#pragma unroll
      for (int q = 0; q < kRsumParts; ++q) {
        t.a += rp[2 * q];
        t.b += rp[2 * q + 1];
      }
      s_rs[tid] = t;
    }
  }
  __syncthreads();
  if (tid == 0) {
    bool resid = job.mode == 2;
    // the chunk sums of the draw's weights
    auto chunk_pair = [&](int ch, bool res) { return res ? s_rs[ch] : Pair{s_zs[ch], 0ull}; };
    Pair tot{0, 0};
    for (int ch = 0; ch < C; ++ch) {
      const Pair q = chunk_pair(ch, resid);
      tot.a += q.a;
      tot.b += q.b;
    }
    if (resid && run_value(c, tot) == 0) {  // p == q at this resolution: draw from p
      resid = false;
      set_mode(c, job, false);
      tot = Pair{0, 0};
      for (int ch = 0; ch < C; ++ch) tot.a += s_zs[ch];
    }
    const u128 t = ((u128)(job.word >> 8) * run_value(c, tot)) >> 24;  // the total < 2^98
    Pair run{0, 0};
    int ch = 0;
    for (; ch < C - 1; ++ch) {
      const Pair q = chunk_pair(ch, resid);
      const Pair nx{run.a + q.a, run.b + q.b};
      if (run_value(c, nx) > t) break;
      run = nx;
    }
    s_ctl[0] = resid;
    s_ctl[1] = ch;
    s_t = t - run_value(c, run);
  }
  __syncthreads();
  set_mode(c, job, s_ctl[0] != 0);
  const int ch = s_ctl[1];
  // read before the scans' barriers: the crossing thread rewrites s_ctl and s_t
  const u128 t = s_t;
  // level 2: the crossing chunk, whole vectors in contiguous runs of `vpt`
  // per thread; the last thread also takes the tail elements
  const int vv0 = ch * a.chunk_vecs, vv1 = min(vv0 + a.chunk_vecs, a.nvec);
  const int vpt = (vv1 - vv0 + kSampDrawThreads - 1) / kSampDrawThreads;  // <= 2
  const int my0 = min(vv0 + tid * vpt, vv1), my1 = min(my0 + vpt, vv1);
  const u32x4* pv = reinterpret_cast<const u32x4*>(c.p);
  const u32x4* qv = reinterpret_cast<const u32x4*>(c.q);
  u32x4 dp[2], dq[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int v = my0 + k;
    dp[k] = v < my1 ? pv[v] : (u32x4){0, 0, 0, 0};
    dq[k] = v < my1 && c.resid ? qv[v] : (u32x4){0, 0, 0, 0};
  }
  const bool last = tid == kSampDrawThreads - 1;
  const int t0 = a.nvec * kEpv;  // first tail element
  const bool has_tail = last && ch == C - 1 && a.tail > 0;
  const bool valid[2] = {my0 < my1, my0 + 1 < my1};
  Pair mine = member_sums<DT, 2>(c, dp, dq, valid);
  if (has_tail) {
    for (int i = t0; i < a.V; ++i) add_elem<DT>(c, i, mine);
  }
  // both exclusive scans with one barrier (each has its own partials)
  unsigned long long tot_a, tot_b;
  const unsigned long long ea =
      block_excl_scan_open<unsigned long long, kSampDrawThreads>(mine.a, s_scan, &tot_a);
  const unsigned long long eb =
      block_excl_scan_open<unsigned long long, kSampDrawThreads>(mine.b, s_scan_b, &tot_b);
  const u128 before = run_value(c, Pair{ea, eb});
  const u128 after = run_value(c, Pair{ea + mine.a, eb + mine.b});
  // exactly one thread has before <= t < after: it hands its element range
  // and what is left of t to wave 0
  if (before <= t && t < after) {
    s_ctl[0] = my0 * kEpv;
    s_ctl[1] = has_tail ? a.V : my1 * kEpv;
    s_t = t - before;
  }
  __syncthreads();
  if (tid >= kWave) return;
  // level 3: one element per lane (at most 2 vectors plus the tail: < 64)
  const int i = s_ctl[0] + tid;
  const bool in = i < s_ctl[1];
  const unsigned int wp = in ? weight(elem<DT>(c.p, i), c.mp, c.cT) : 0u;
  const unsigned int wq = in && c.resid ? weight(elem<DT>(c.q, i), c.mq, c.cT) : 0u;
  const bool mem = in && member(c, wp, wq);
  const unsigned long long ia = wave_incl_scan_op(mem ? (unsigned long long)wp : 0ull, 0ull, OpAdd{});
  const unsigned long long ib = wave_incl_scan_op(mem ? (unsigned long long)wq : 0ull, 0ull, OpAdd{});
  const unsigned long long cross = __ballot(in && run_value(c, Pair{ia, ib}) > s_t);
  if (tid == 0) {
    const int tok = s_ctl[0] + (cross ? __builtin_ctzll(cross) : 0);
    a.bonus[r] = tok;
    a.out_tokens[(size_t)r * (a.gamma + 1) + job.col] = tok;
  }
}

template <dspark_dtype DT>
hipError_t launch_rowstat(const SampArgs& a, int grid, hipStream_t s) {
  const int slots = (a.nvec + kRsThreads - 1) / kRsThreads;
  if (slots <= 2) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(samp_rowstat_kernel<DT, 2>), dim3(grid), dim3(kRsThreads), 0, s, a);
  } else if (slots <= 4) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(samp_rowstat_kernel<DT, 4>), dim3(grid), dim3(kRsThreads), 0, s, a);
  } else if (slots <= 8) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(samp_rowstat_kernel<DT, 8>), dim3(grid), dim3(kRsThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(samp_rowstat_kernel<DT, 16>), dim3(grid), dim3(kRsThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <dspark_dtype DT>
hipError_t launch_dt(SampArgs a, hipStream_t s) {
  const long long units = (long long)a.B * (2 * a.gamma + 1) * a.chunks;
  // rows of 1024 to 16384 vectors take the one-read row-statistics kernel:
  // one persistent workgroup per CU, at most kRsMaxList rows each. Every
  // workgroup scans all the slots to find its rows, so larger batches (more
  // than kRsMaxList slots per CU) keep the two-read kernels.
  int grid = 0;
  if (a.B > 0 && a.nvec >= kRsThreads && a.nvec <= kRsMaxSlots * kRsThreads) {
    int cus = 1;
    hipError_t e = current_cu_count(&cus);
    if (e != hipSuccess) return e;
    const long long slots = (long long)a.B * (2 * a.gamma + 1);
    const int g = (int)std::min<long long>(cus, slots);
    // each thread keeps the liveness of at most 64 slots as bits
    if (slots <= (long long)kRsMaxList * g && slots <= 64LL * kRsThreads) grid = g;
  }
  a.rowstat = grid > 0;
  hipError_t e;
  if (a.rowstat) {
    e = launch_rowstat<DT>(a, grid, s);
  } else {
    hipLaunchKernelGGL(samp_max_kernel<DT>, dim3(units > 0 ? (unsigned)units : 1u),
                       dim3(kSampThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.B == 0) return e;
    hipLaunchKernelGGL(samp_z_kernel<DT>, dim3((unsigned)units), dim3(kSampThreads), 0, s, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(samp_decide_kernel<DT>, dim3(a.B), dim3(kWave), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(samp_rsum_kernel<DT>, dim3((unsigned)(a.B * a.chunks * kRsumParts)),
                     dim3(kSampThreads), 0, s, a);
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
