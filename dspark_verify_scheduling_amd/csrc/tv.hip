// Soft accept-rate a = 1 - TV(softmax q, softmax p) and its cumulative
// product per request.
//
// Method source: "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §二
// (DeepSpec accept_rate = 1 - 0.5 * sum |draft_probs - target_probs|, which
// equals sum_x min(p(x), q(x)) under rejection sampling, and
// confidence_prefix_targets = accept_rate.cumprod).
//
// Computation. With log-partitions A_q = max q + ln sum e^(q - max q) (and the
// same for p), min(u_x, v_x) = exp(min(q_x - A_q, p_x - A_p)). So
// a = sum_x exp(min(q_x - A_q, p_x - A_p)) needs one exponential per element
// pair once the partitions are known:
//   pass 1: online (max, sum-exp) of q and of p, per thread, merged over the
//           workgroup;
//   pass 2: the sum of exp(min(...)). The pair's rows (about 0.5 MB at
//           V = 129280 bf16) were just read, so the re-read is served mostly
//           from the caches.
// Exponentials are exp2 of base-2 scaled values (hardware v_exp_f32). The
// result is clamped to at most 1; rounding can exceed 1 by ~1e-7.
#include <float.h>

#include "common.h"

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWaves = kTvThreads / kWave;

template <dspark_dtype DT>
__device__ inline void widen(const u32x4& d, float* x) {
  if constexpr (DT == DSPARK_BF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = __uint_as_float(d[w] << 16);
      x[2 * w + 1] = __uint_as_float(d[w] & 0xFFFF0000u);
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

struct MS {
  float m, s;  // running max and sum of exp2(y - m), y in base-2 units
};

__device__ inline MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  return {m, a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m)};
}

template <int N>
__device__ inline void ms_add(MS& st, const float* x) {
  float y[N];
  float mloc = st.m;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    y[i] = x[i] * kLog2e;
    mloc = fmaxf(mloc, y[i]);
  }
  float acc = st.s * exp2f(st.m - mloc);
#pragma unroll
  for (int i = 0; i < N; ++i) acc += exp2f(y[i] - mloc);
  st = {mloc, acc};
}

__device__ inline MS block_ms(MS v, float* sm, float* ss) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    MS o{__shfl_xor(v.m, off, kWave), __shfl_xor(v.s, off, kWave)};
    v = ms_merge(v, o);
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (lane == 0) {
    sm[wave] = v.m;
    ss[wave] = v.s;
  }
  __syncthreads();
  MS t{sm[0], ss[0]};
  for (int w = 1; w < kWaves; ++w) t = ms_merge(t, MS{sm[w], ss[w]});
  __syncthreads();
  return t;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kTvThreads) void tv_kernel(TvArgs a) {
  __shared__ float sm[kWaves], ss[kWaves];
  __shared__ float sd[kWaves];
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  const int pair = blockIdx.x;
  const int r = pair / a.gamma;
  const int k0 = pair - r * a.gamma;
  const unsigned char* qrow = a.q + (size_t)pair * a.ldq_bytes;
  const unsigned char* prow = a.p + ((size_t)r * a.rows_per_req + k0) * a.ldp_bytes;
  const u32x4* qv = reinterpret_cast<const u32x4*>(qrow);
  const u32x4* pv = reinterpret_cast<const u32x4*>(prow);
  const int tid = threadIdx.x;

  // pass 1: log-partitions
  MS sq{-FLT_MAX, 0.0f}, sp{-FLT_MAX, 0.0f};
  for (int v = tid; v < a.nvec; v += kTvThreads) {
    const u32x4 dq = qv[v], dp = pv[v];
    float x[kEpv];
    widen<DT>(dq, x);
    ms_add<kEpv>(sq, x);
    widen<DT>(dp, x);
    ms_add<kEpv>(sp, x);
  }
  if (tid == 0) {
    for (int t = 0; t < a.tail; ++t) {
      const int i = a.nvec * kEpv + t;
      float x = elem<DT>(qrow, i);
      ms_add<1>(sq, &x);
      x = elem<DT>(prow, i);
      ms_add<1>(sp, &x);
    }
  }
  sq = block_ms(sq, sm, ss);
  sp = block_ms(sp, sm, ss);
  const float aq = sq.m + log2f(sq.s);  // base-2 log-partitions
  const float ap = sp.m + log2f(sp.s);

  // pass 2: sum of min(u, v)
  float acc = 0.0f;
  for (int v = tid; v < a.nvec; v += kTvThreads) {
    const u32x4 dq = __builtin_nontemporal_load(qv + v);
    const u32x4 dp = __builtin_nontemporal_load(pv + v);
    float xq[kEpv], xp[kEpv];
    widen<DT>(dq, xq);
    widen<DT>(dp, xp);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < kEpv; ++i) {
      part += exp2f(fminf(xq[i] * kLog2e - aq, xp[i] * kLog2e - ap));
    }
    acc += part;
  }
  if (tid == 0) {
    for (int t = 0; t < a.tail; ++t) {
      const int i = a.nvec * kEpv + t;
      acc += exp2f(fminf(elem<DT>(qrow, i) * kLog2e - aq, elem<DT>(prow, i) * kLog2e - ap));
    }
  }
  const float total = block_sum<float, kTvThreads>(acc, sd);
  if (tid == 0) a.a_out[pair] = total > 1.0f ? 1.0f : total;
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
    if (dt == DSPARK_BF16) {
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
