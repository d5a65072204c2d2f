// Soft accept-rate a = 1 - TV(softmax q, softmax p) and its cumulative
// product per request.
//
// Method source: "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §二
// (DeepSpec accept_rate = 1 - 0.5 * sum |draft_probs - target_probs|, which
// equals sum_x min(p(x), q(x)) under rejection sampling, and
// confidence_prefix_targets = accept_rate.cumprod).
//
// Computation. With base-2 log-partitions A_q = log2 sum_x 2^(q_x log2 e) (and
// the same for p), min(u_x, v_x) = 2^min(q_x log2 e - A_q, p_x log2 e - A_p),
// so a = sum_x 2^min(...) needs one exponential per element pair once the
// partitions are known. Two passes over each (draft row, target row) pair:
//   pass 1: each thread's (offset, sum of 2^(x log2 e - offset)) of each row;
//           the workgroup merges the threads' into A_q and A_p;
//   pass 2: the sum of 2^min(...) over the same rows.
// Rows that fit on one CU (bf16 V up to 130055) take tv_resident_kernel: one
// persistent workgroup per CU keeps each pair in registers and LDS between
// the passes, so every logit is read from HBM once, and loads the next pair
// while it finishes the current one. The same kernel takes rows of up to
// 4096 vectors more (bf16 V up to 162823) and reads only those vectors twice.
// Longer rows take tv_kernel, one
// workgroup per pair, which streams them twice (pass 1 with ordinary loads,
// pass 2 with nontemporal ones); the pair's rows are then mostly gone from the
// XCD's 4 MB L2 when pass 2 comes back to them.
// Exponentials are the raw v_exp_f32 (exp2 without the denormal-range fix-up:
// results below 2^-126 are negligible in a sum that is about 1). The result is
// clamped to at most 1; rounding can exceed 1 by ~1e-7.
#include <float.h>

#include "common.h"

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWaves = kTvThreads / kWave;
constexpr int kU = 4;  // vectors of q (and of p) per thread per batch

__device__ inline float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

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

template <dspark_dtype DT>
__device__ inline float elem(const unsigned char* row, int i) {
  if constexpr (DT == DSPARK_BF16) {
    return __uint_as_float((unsigned int)reinterpret_cast<const unsigned short*>(row)[i] << 16);
  } else {
    return reinterpret_cast<const float*>(row)[i];
  }
}

// Partial log-partition state in base-2 units: s = sum 2^(x log2 e - mL)
// over the elements seen, mL >= -FLT_MAX finite (so -inf inputs and empty
// states stay finite). The streaming kernel keeps mL at the running maximum;
// the resident kernel uses a fixed offset per thread.
struct Stat {
  float mL, s;
};

__device__ inline Stat stat_merge(Stat a, Stat b) {
  const float m = fmaxf(a.mL, b.mL);
  return {m, a.s * exp2_raw(a.mL - m) + b.s * exp2_raw(b.mL - m)};
}

// Adds N values whose maximum is bm.
template <int N>
__device__ inline void stat_add(Stat& st, const float* x, float bm) {
  const float mL = fmaxf(st.mL, fmaxf(bm * kLog2e, -FLT_MAX));
  float acc0 = st.s * exp2_raw(st.mL - mL), acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    acc0 += exp2_raw(__fmaf_rn(x[i], kLog2e, -mL));
    acc1 += exp2_raw(__fmaf_rn(x[i + 1], kLog2e, -mL));
  }
  st = {mL, acc0 + acc1};
}

__device__ inline Stat block_stat(Stat v, Stat* ws) {
  const Stat ident{-FLT_MAX, 0.0f};
  auto op = [](Stat a, Stat b) { return stat_merge(a, b); };
  return block_reduce<Stat, kTvThreads>(v, ident, op, ws);
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kTvThreads) void tv_kernel(TvArgs a) {
  __shared__ Stat ws[kWaves];
  __shared__ float wsf[kWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  constexpr int kN = kU * kEpv;  // values of one row per thread per batch
  // -inf in every lane: no effect on a maximum, 2^-inf = 0 in a sum
  constexpr unsigned int kNegInf = DT == DSPARK_BF16 ? 0xFF80FF80u : 0xFF800000u;
  const int pair = blockIdx.x;
  const int r = pair / a.gamma;
  const int k0 = pair - r * a.gamma;
  const unsigned char* qrow = a.q + (size_t)pair * a.ldq_bytes;
  const unsigned char* prow = a.p + ((size_t)r * a.rows_per_req + k0) * a.ldp_bytes;
  const u32x4* qv = reinterpret_cast<const u32x4*>(qrow);
  const u32x4* pv = reinterpret_cast<const u32x4*>(prow);
  const int tid = threadIdx.x;
  const u32x4 fill = (u32x4){kNegInf, kNegInf, kNegInf, kNegInf};

  // pass 1: log-partitions
  Stat sq{-FLT_MAX, 0.0f}, sp{-FLT_MAX, 0.0f};
  for (int v0 = tid; v0 < a.nvec; v0 += kTvThreads * kU) {
    u32x4 dq[kU], dp[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kTvThreads;
      dq[u] = fill;
      dp[u] = fill;
      if (v < a.nvec) {
        dq[u] = qv[v];
        dp[u] = pv[v];
      }
    }
    float x[kN], y[kN];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      widen<DT>(dq[u], x + u * kEpv);
      widen<DT>(dp[u], y + u * kEpv);
    }
    float bq = x[0], bp = y[0];
#pragma unroll
    for (int i = 1; i < kN; ++i) {
      bq = fmaxf(bq, x[i]);
      bp = fmaxf(bp, y[i]);
    }
    stat_add<kN>(sq, x, bq);
    stat_add<kN>(sp, y, bp);
  }
  if (tid == 0) {
    for (int t = 0; t < a.tail; ++t) {
      const int i = a.nvec * kEpv + t;
      float x[2] = {elem<DT>(qrow, i), -INFINITY};
      stat_add<2>(sq, x, x[0]);
      float y[2] = {elem<DT>(prow, i), -INFINITY};
      stat_add<2>(sp, y, y[0]);
    }
  }
  sq = block_stat(sq, ws);
  sp = block_stat(sp, ws);
  const float aq = sq.mL + log2f(sq.s);  // base-2 log-partitions
  const float ap = sp.mL + log2f(sp.s);

  // pass 2: sum of min(u, v)
  float acc0 = 0.0f, acc1 = 0.0f;
  for (int v0 = tid; v0 < a.nvec; v0 += kTvThreads * kU) {
    u32x4 dq[kU], dp[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kTvThreads;
      dq[u] = fill;
      dp[u] = fill;
      if (v < a.nvec) {
        dq[u] = __builtin_nontemporal_load(qv + v);
        dp[u] = __builtin_nontemporal_load(pv + v);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float x[kEpv], y[kEpv];
      widen<DT>(dq[u], x);
      widen<DT>(dp[u], y);
#pragma unroll
      for (int i = 0; i < kEpv; i += 2) {
        acc0 += exp2_raw(fminf(__fmaf_rn(x[i], kLog2e, -aq), __fmaf_rn(y[i], kLog2e, -ap)));
        acc1 += exp2_raw(
            fminf(__fmaf_rn(x[i + 1], kLog2e, -aq), __fmaf_rn(y[i + 1], kLog2e, -ap)));
      }
    }
  }
  float acc = acc0 + acc1;
  if (tid == 0) {
    for (int t = 0; t < a.tail; ++t) {
      const int i = a.nvec * kEpv + t;
      acc += exp2_raw(fminf(__fmaf_rn(elem<DT>(qrow, i), kLog2e, -aq),
                            __fmaf_rn(elem<DT>(prow, i), kLog2e, -ap)));
    }
  }
  const float total = block_sum<float, kTvThreads>(acc, wsf);
  if (tid == 0) a.a_out[pair] = total > 1.0f ? 1.0f : total;
}

// Sum of 2^(x log2 e - off) over one row's 16 bytes.
template <dspark_dtype DT>
__device__ inline float exp_sum_vec(const u32x4& d, float off) {
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  float x[kEpv];
  widen<DT>(d, x);
  // the partial sums start at their first term, not at 0 + that term (the
  // same value: exponentials are >= +0), which the compiler would keep as an
  // add
  float s0 = exp2_raw(__fmaf_rn(x[0], kLog2e, -off));
  float s1 = exp2_raw(__fmaf_rn(x[1], kLog2e, -off));
#pragma unroll
  for (int i = 2; i < kEpv; i += 2) {
    s0 += exp2_raw(__fmaf_rn(x[i], kLog2e, -off));
    s1 += exp2_raw(__fmaf_rn(x[i + 1], kLog2e, -off));
  }
  return s0 + s1;
}

// Maximum of one row's 16 bytes (NaN ignored).
template <dspark_dtype DT>
__device__ inline float vec_max(const u32x4& d) {
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  float x[kEpv];
  widen<DT>(d, x);
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < kEpv; ++i) bm = fmaxf(bm, x[i]);
  return bm;
}

// The offset of a thread's fixed-offset sums: the maximum of its first
// vector (base-2 units), finite.
template <dspark_dtype DT>
__device__ inline float first_offset(const u32x4& d) {
  return fmaxf(vec_max<DT>(d) * kLog2e, -FLT_MAX);
}

template <dspark_dtype DT>
__device__ inline float min_sum_pair(const u32x4& dq, const u32x4& dp, float aq, float ap) {
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  float x[kEpv], y[kEpv];
  widen<DT>(dq, x);
  widen<DT>(dp, y);
  // started at the first terms, as in exp_sum_vec
  float s0 = exp2_raw(fminf(__fmaf_rn(x[0], kLog2e, -aq), __fmaf_rn(y[0], kLog2e, -ap)));
  float s1 = exp2_raw(fminf(__fmaf_rn(x[1], kLog2e, -aq), __fmaf_rn(y[1], kLog2e, -ap)));
#pragma unroll
  for (int i = 2; i < kEpv; i += 2) {
    s0 += exp2_raw(fminf(__fmaf_rn(x[i], kLog2e, -aq), __fmaf_rn(y[i], kLog2e, -ap)));
    s1 += exp2_raw(fminf(__fmaf_rn(x[i + 1], kLog2e, -aq), __fmaf_rn(y[i + 1], kLog2e, -ap)));
  }
  return s0 + s1;
}

// Direct global-to-LDS copy of one wave's 64 x 16 bytes: lane l's vector
// src[l] lands at LDS byte address lds_addr + 16 l, without passing through
// registers. src and lds_addr are wave-uniform (SGPR base address, the lane's
// byte offset in a VGPR); M0 holds lds_addr (one wait state before the load
// reads it; nothing else in these kernels uses M0, so it is not saved). Written
// as inline assembly so that the compiler's wait-count bookkeeping does not
// see it: its waits for the register loads stay exact positions in the load
// queue (the copies only make them more conservative), and the callers wait
// for the copies themselves (vmcnt(0) and a barrier) before reading the LDS.
__device__ inline void lds_dma16(const u32x4* src, unsigned int lds_addr, unsigned int lane_bytes) {
  const unsigned long long g = (unsigned long long)src;
  const unsigned long long g_uniform =
      ((unsigned long long)(unsigned int)__builtin_amdgcn_readfirstlane((int)(g >> 32)) << 32) |
      (unsigned int)__builtin_amdgcn_readfirstlane((int)(unsigned int)g);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_bytes), "s"(g_uniform), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

__device__ inline void pair_rows(const TvArgs& a, int pair, const u32x4*& qv, const u32x4*& pv) {
  const int r = pair / a.gamma;
  const int k0 = pair - r * a.gamma;
  qv = reinterpret_cast<const u32x4*>(a.q + (size_t)pair * a.ldq_bytes);
  pv = reinterpret_cast<const u32x4*>(a.p + ((size_t)r * a.rows_per_req + k0) * a.ldp_bytes);
}

struct OpMaxF {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Wave-wide merge of a Stat on DPP lane exchanges (no LDS, no address
// registers); the result is uniform over the wave.
__device__ inline Stat wave_stat(Stat st) {
  const float m = read_lane(wave_incl_scan_op(st.mL, -FLT_MAX, OpMaxF{}), kWave - 1);
  const float s = read_lane(wave_incl_scan_op(st.s * exp2_raw(st.mL - m), 0.0f, OpAdd{}), kWave - 1);
  return {m, s};
}

__device__ inline float wave_total(float v) {
  return read_lane(wave_incl_scan_op(v, 0.0f, OpAdd{}), kWave - 1);
}

// Both rows' statistics merged over the workgroup in one round: each wave
// merges its lanes', lane w of every wave then reads wave w's and merges
// those. Every thread returns with the workgroup's statistics.
__device__ inline void block_stat2(Stat& sq, Stat& sp, float4* ws) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  sq = wave_stat(sq);
  sp = wave_stat(sp);
  if (lane == 0) ws[wave] = make_float4(sq.mL, sq.s, sp.mL, sp.s);
  __syncthreads();
  const float4 w = lane < kWaves ? ws[lane] : make_float4(-FLT_MAX, 0.0f, -FLT_MAX, 0.0f);
  sq = wave_stat({w.x, w.y});
  sp = wave_stat({w.z, w.w});
}

// Resident, persistent variant: one workgroup per CU walks the pairs
// blockIdx.x, blockIdx.x + gridDim.x, ..., keeping each pair on the CU between
// the passes so that every logit is read from HBM once. Vector pair v (16
// bytes of q and of p) lives
//   in registers of thread v % 1024 (slot v / 1024) for v < 11 * 1024, and
//   in LDS for the rest (q at i, p at n_lds + i, i = v - 11 * 1024),
// which holds rows of up to 11 * 1024 + 4992 vectors (bf16 V <= 130055):
// 88 VGPRs and up to 156 KB of LDS. Up to kResMaxOverflow vectors past those
// are read from memory twice: in pass 1 after the LDS part, and in pass 2
// before the register slots (so that waiting for them never waits for the
// next pair's reloads). The next pair's loads are issued while pass 2 of the
// current one runs: each register slot is reloaded as soon as pass 2 has
// consumed it, and the LDS part is copied straight from HBM into LDS (no
// registers) once every wave has read the current one. Pass 1 of the next
// pair then consumes the slots in the order they arrive.
//
// FULL (rows of at least 11 * 1024 vectors) issues every register-slot load
// unconditionally, so the compiler can wait for each slot by its position in
// the load queue instead of for the whole queue; after the last pair the
// reloads read the current row's first 1 KB again (cached), and are unused.
// Shorter rows fill the slots past the row end with -inf instead. Rows past
// the overflow limit take the two-pass streaming kernel above.
constexpr int kResRegSlots = 11;
constexpr int kResLdsSlots = 5;
constexpr int kResRegSpan = kResRegSlots * kTvThreads;
constexpr int kResLdsMaxPairs = 4992;  // 2 * 4992 * 16 B = 156 KB
// vectors past the register slots and the LDS part (read twice, from memory):
// rows of up to 11 * 1024 + 4992 + 4096 vectors (bf16 V <= 162823)
constexpr int kResMaxOverflow = 4 * kTvThreads;

template <dspark_dtype DT, bool FULL>
__global__ __launch_bounds__(kTvThreads) void tv_resident_kernel(TvArgs a) {
  extern __shared__ u32x4 lds_pairs[];  // q vectors [n_lds], then p vectors [n_lds]
  __shared__ float4 ws[kWaves];
  __shared__ float wsf[kWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  constexpr unsigned int kNegInf = DT == DSPARK_BF16 ? 0xFF80FF80u : 0xFF800000u;
  const int pairs = a.B * a.gamma;
  const int tid = threadIdx.x;
  const int wave_off = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));
  const unsigned int lane_bytes = (unsigned int)(tid & (kWave - 1)) * sizeof(u32x4);
  const int nvec = a.nvec;
  const int n_lds = FULL ? min(nvec - kResRegSpan, kResLdsMaxPairs) : 0;
  // The overflow vectors [x0, nvec), read twice. Thread tid takes those
  // congruent to tid modulo the workgroup size, starting at xs, as in the
  // register slots and the LDS part: the rare exact re-sum of pass 1 sweeps
  // v = tid, tid + 1024, ... and so covers the same vectors.
  const int x0 = kResRegSpan + n_lds;
  const int xs = x0 + ((tid - x0) & (kTvThreads - 1));
  u32x4* lq = lds_pairs;
  u32x4* lp = lds_pairs + n_lds;
  // LDS byte addresses of the two parts (uniform), for the copies
  const unsigned int lq_addr = (unsigned int)__builtin_amdgcn_readfirstlane(
      (int)(unsigned int)(size_t)(__attribute__((address_space(3))) void*)lds_pairs);
  const unsigned int lp_addr = lq_addr + (unsigned int)n_lds * 16u;
  const u32x4 fill = (u32x4){kNegInf, kNegInf, kNegInf, kNegInf};

  int pair = blockIdx.x;
  const u32x4 *qv, *pv;
  pair_rows(a, pair, qv, pv);
  u32x4 rq[kResRegSlots], rp[kResRegSlots];
#pragma unroll
  for (int c = 0; c < kResRegSlots; ++c) {
    const int v = c * kTvThreads + tid;
    if (FULL) {
      // issued in slot order, the order pass 1 consumes them in
      rq[c] = qv[v];
      rp[c] = pv[v];
      __builtin_amdgcn_sched_barrier(0);
    } else {
      rq[c] = fill;
      rp[c] = fill;
      if (v < nvec) {
        rq[c] = qv[v];
        rp[c] = pv[v];
      }
    }
  }
  if (FULL) {
#pragma unroll
    for (int c = 0; c < kResLdsSlots; ++c) {
      const int i = c * kTvThreads + tid;
      if (i < n_lds) {
        const int w0 = c * kTvThreads + wave_off;
        lds_dma16(qv + kResRegSpan + w0, lq_addr + w0 * 16u, lane_bytes);
        lds_dma16(pv + kResRegSpan + w0, lp_addr + w0 * 16u, lane_bytes);
      }
    }
  }

  for (;;) {
    const unsigned char* qrow = reinterpret_cast<const unsigned char*>(qv);
    const unsigned char* prow = reinterpret_cast<const unsigned char*>(pv);
    // pass 1: register slots in arrival order, then (every wave's copies
    // complete) the LDS part. Each thread sums 2^(x log2 e - off) with one
    // offset per row, the maximum of its first vector: no running maximum and
    // no rescaling. A lane whose sums overflow (an element about 2^7 or more
    // above that maximum in base-2 units, or non-finite data) sums again with
    // its exact maximum as the offset.
    auto row_sums = [&](float oq, float op, float& fq, float& fp) {
      fq = 0.0f;
      fp = 0.0f;
#pragma unroll
      for (int c = 0; c < kResRegSlots; ++c) {
        fq += exp_sum_vec<DT>(rq[c], oq);
        fp += exp_sum_vec<DT>(rp[c], op);
      }
      if (tid == 0) {
        for (int t = 0; t < a.tail; ++t) {
          const int i = nvec * kEpv + t;
          fq += exp2_raw(__fmaf_rn(elem<DT>(qrow, i), kLog2e, -oq));
          fp += exp2_raw(__fmaf_rn(elem<DT>(prow, i), kLog2e, -op));
        }
      }
    };
    auto lds_sums = [&](float oq, float op, float& fq, float& fp) {
#pragma unroll
      for (int c = 0; c < kResLdsSlots; ++c) {
        const int i = c * kTvThreads + tid;
        if (i < n_lds) {
          fq += exp_sum_vec<DT>(lq[i], oq);
          fp += exp_sum_vec<DT>(lp[i], op);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    float oq = first_offset<DT>(rq[0]);
    float op = first_offset<DT>(rp[0]);
    float fq, fp;
    row_sums(oq, op, fq, fp);
    if (FULL) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      lds_sums(oq, op, fq, fp);
#pragma unroll 1
      for (int v = xs; v < nvec; v += kTvThreads) {  // overflow, first read
        fq += exp_sum_vec<DT>(qv[v], oq);
        fp += exp_sum_vec<DT>(pv[v], op);
      }
    }
    if (!(fq <= FLT_MAX && fp <= FLT_MAX)) {
      // rare: two sweeps over this thread's vectors, read again from memory
      float mq = -FLT_MAX, mp = -FLT_MAX;
#pragma unroll 1
      for (int v = tid; v < nvec; v += kTvThreads) {
        mq = fmaxf(mq, vec_max<DT>(qv[v]));
        mp = fmaxf(mp, vec_max<DT>(pv[v]));
      }
      if (tid == 0) {
        for (int t = 0; t < a.tail; ++t) {
          const int i = nvec * kEpv + t;
          mq = fmaxf(mq, elem<DT>(qrow, i));
          mp = fmaxf(mp, elem<DT>(prow, i));
        }
      }
      oq = fmaxf(mq * kLog2e, -FLT_MAX);
      op = fmaxf(mp * kLog2e, -FLT_MAX);
      fq = 0.0f;
      fp = 0.0f;
#pragma unroll 1
      for (int v = tid; v < nvec; v += kTvThreads) {
        fq += exp_sum_vec<DT>(qv[v], oq);
        fp += exp_sum_vec<DT>(pv[v], op);
      }
      if (tid == 0) {
        for (int t = 0; t < a.tail; ++t) {
          const int i = nvec * kEpv + t;
          fq += exp2_raw(__fmaf_rn(elem<DT>(qrow, i), kLog2e, -oq));
          fp += exp2_raw(__fmaf_rn(elem<DT>(prow, i), kLog2e, -op));
        }
      }
    }
    Stat sq{oq, fq}, sp{op, fp};
    block_stat2(sq, sp, ws);
    const float aq = sq.mL + log2f(sq.s);  // base-2 log-partitions
    const float ap = sp.mL + log2f(sp.s);

    // pass 2: the tail and any overflow vectors first (their loads are then
    // not queued behind the reloads), then the register slots, each reloaded
    // with the next pair once consumed, then the LDS part. The empty asm
    // makes the raw words opaque, so pass 2 widens them again instead of
    // keeping pass 1's fp32 copies alive.
    float acc = 0.0f;
    if (tid == 0) {
      for (int t = 0; t < a.tail; ++t) {
        const int i = nvec * kEpv + t;
        acc += exp2_raw(fminf(__fmaf_rn(elem<DT>(qrow, i), kLog2e, -aq),
                              __fmaf_rn(elem<DT>(prow, i), kLog2e, -ap)));
      }
    }
    if (FULL) {
#pragma unroll 1
      for (int v = xs; v < nvec; v += kTvThreads)  // overflow, second read
        acc += min_sum_pair<DT>(qv[v], pv[v], aq, ap);
    }
    const int next = pair + gridDim.x;
    const bool more = next < pairs;
    const u32x4 *nqv = qv, *npv = pv;
    if (more) pair_rows(a, next, nqv, npv);
#pragma unroll
    for (int c = 0; c < kResRegSlots; ++c) asm volatile("" : "+v"(rq[c]), "+v"(rp[c]));
#pragma unroll
    for (int c = 0; c < kResRegSlots; ++c) {
      acc += min_sum_pair<DT>(rq[c], rp[c], aq, ap);
      // The reload's address depends on this opaque copy of the thread index,
      // tied to acc, so the slot's old words are consumed before it is issued.
      int lt = tid;
      asm volatile("" : "+v"(lt), "+v"(acc));
      const int v = c * kTvThreads + lt;
      if (FULL) {
        const int vl = more ? v : (lt & (kWave - 1));
        rq[c] = nqv[vl];
        rp[c] = npv[vl];
      } else {
        rq[c] = fill;
        rp[c] = fill;
        if (more && v < nvec) {
          rq[c] = nqv[v];
          rp[c] = npv[v];
        }
      }
    }
    if (FULL) {
#pragma unroll
      for (int c = 0; c < kResLdsSlots; ++c) {
        const int i = c * kTvThreads + tid;
        if (i < n_lds) acc += min_sum_pair<DT>(lq[i], lp[i], aq, ap);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    acc = wave_total(acc);
    if (lane_id() == 0) wsf[tid / kWave] = acc;
    // after this barrier no wave reads the LDS part any more
    __syncthreads();
    if (FULL && more) {
      // opaque copies of the wave offset and the LDS addresses: the compiler
      // would otherwise share the per-slot offsets with the first copies
      // before the loop, where they are defined under the lane condition and
      // so are kept in VGPRs
      unsigned int qa = lq_addr, pa = lp_addr;
      int wo = wave_off;
      asm volatile("" : "+s"(qa), "+s"(pa), "+s"(wo));
#pragma unroll
      for (int c = 0; c < kResLdsSlots; ++c) {
        const int i = c * kTvThreads + tid;
        if (i < n_lds) {
          const int w0 = c * kTvThreads + wo;
          lds_dma16(nqv + kResRegSpan + w0, qa + w0 * 16u, lane_bytes);
          lds_dma16(npv + kResRegSpan + w0, pa + w0 * 16u, lane_bytes);
        }
      }
    }
    if (tid == 0) {
      float total = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) total += wsf[w];
      a.a_out[pair] = total > 1.0f ? 1.0f : total;
    }
    if (!more) break;
    pair = next;
    qv = nqv;
    pv = npv;
  }
}

__global__ void tv_cumprod_kernel(const float* a_in, float* s_out, int B, int G) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  float s = 1.0f;
  for (int k = 0; k < G; ++k) {
    const float v = a_in[(size_t)r * G + k];
    s = k == 0 ? v : __fmul_rn(s, v);
    s_out[(size_t)r * G + k] = s;
  }
}

}  // namespace

hipError_t launch_tv(const TvArgs& a, dspark_dtype dt, hipStream_t s) {
  const int pairs = a.B * a.gamma;
  if (pairs > 0) {
    const int n_rest = a.nvec > kResRegSpan ? a.nvec - kResRegSpan : 0;
    const int n_lds = n_rest < kResLdsMaxPairs ? n_rest : kResLdsMaxPairs;
    if (n_rest - n_lds <= kResMaxOverflow) {
      // one persistent workgroup per CU (the registers hold one per CU)
      int cus = 1;
      hipError_t e = current_cu_count(&cus);
      if (e != hipSuccess) return e;
      const int grid = pairs < cus ? pairs : cus;
      const size_t lds = (size_t)2 * n_lds * sizeof(u32x4);
      const bool full = n_lds > 0 || a.nvec == kResRegSpan;
      void (*kern)(TvArgs);
      if (dt == DSPARK_BF16) {
        kern = full ? tv_resident_kernel<DSPARK_BF16, true> : tv_resident_kernel<DSPARK_BF16, false>;
      } else {
        kern = full ? tv_resident_kernel<DSPARK_F32, true> : tv_resident_kernel<DSPARK_F32, false>;
      }
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kTvThreads), lds, s, a);
    } else if (dt == DSPARK_BF16) {
      hipLaunchKernelGGL(tv_kernel<DSPARK_BF16>, dim3(pairs), dim3(kTvThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(tv_kernel<DSPARK_F32>, dim3(pairs), dim3(kTvThreads), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int threads = 256;
    hipLaunchKernelGGL(tv_cumprod_kernel, dim3((a.B + threads - 1) / threads), dim3(threads), 0, s,
                       (const float*)a.a_out, a.s_out, a.B, a.gamma);
  }
  return hipGetLastError();
}

}  // namespace dspark
