// Greedy accept: per-row argmax over the packed target logits, then the
// per-request leading-match count, bonus, commit and output tokens.
//
// Method sources:
//   "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit" (akiyangdev)
//     §四: verify row j's prediction checks draft j+1 (R checks A, A checks B);
//     §五: AcceptGreedy (target_predict = argmax, correct_len = leading
//          matches, bonus = prediction of the last valid input row),
//          FinalizeAcceptLens (commit = correct + 1, new_seq = prefix +
//          commit), BuildOutTokens (copy drafts, scatter bonus at correct).
//   "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev) §二: prefix_mask =
//     positions < num_correct_drafts; a match after the first mismatch is
//     not accepted.
//
// Two kernels on the caller's stream:
//
// 1. accept_argmax_kernel streams the total * V logits once. One
//    256-thread workgroup per (row, unit) of up to 2048 16-byte vectors
//    (32 KB); eight nontemporal 16-byte loads per thread are in flight before
//    any arithmetic. For bf16 the common case costs two packed 16-bit
//    instructions per pair of elements: a signed max of the raw bits (the
//    order of non-negative bf16 values) and an unsigned max that detects
//    negative NaNs. When the unit's maximum is positive and it holds no NaN,
//    only the lanes that hold the maximum search their registers for its
//    first position. Otherwise the unit is redone exactly from the same
//    registers with a total-order key (NaN highest, -0 == +0, lowest index
//    wins). Each unit writes one 64-bit (key, index) partial. The kernel has
//    no atomics and no cross-workgroup waits.
// 2. accept_finalize_kernel: one wave per request merges its rows' partials,
//    counts the leading matches with a ballot, and writes the outputs; a
//    grid-stride pass writes the row argmax of every packed row.
//
// Cap-accept ("DSpark接入SGLang：用置信度驱动可变长度验证" (yingzheng), the
// three verify modes and the observability section; "DSpark 自适应 Verify
// 怎样分配候选预算" §五, cap-accept) runs the same two kernels on the fixed
// strided layout of B * (gamma + 1) rows: the leading matches are counted
// over all gamma drafts (the ceiling), then clipped to verify_len - 1, which
// commits what compact mode commits.
//
// The partials are fully rewritten by every call, so the workspace needs no
// initialization and holds no state between calls.
#include "common.h"

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = kAccThreads / kWave;

// Reinterpret a dword as two 16-bit lanes. The dword is taken by value: with
// this toolchain, __builtin_bit_cast applied directly to an ext_vector element
// (d[j][w]) reads element 0 of the vector whatever the subscript.
__device__ inline i16x2 as_i16x2(unsigned int x) { return __builtin_bit_cast(i16x2, x); }
__device__ inline u16x2 as_u16x2(unsigned int x) { return __builtin_bit_cast(u16x2, x); }

// 16-bit order key of two bf16 values packed in one dword (each half
// independently): larger value -> larger key; -0 == +0; NaN above +inf.
//   m = sign mask (0xFFFF for negatives); (h ^ (m | 0x8000)) - m maps the
//   sign-magnitude bits to an order-preserving integer (-0 and +0 both to
//   0x8000, -inf to 0x0080). Subtracting 0x80 moves -inf to 0 and every NaN to
//   0xFF01..0xFFFF (wrapping); the final min folds all NaNs onto 0xFF01.
//   A positive non-NaN h maps to h + 0x7F80.
__device__ inline unsigned int bf16x2_keys(unsigned int w) {
  const i16x2 v = __builtin_bit_cast(i16x2, w);
  const i16x2 m = v >> (i16x2){15, 15};
  const unsigned int mu = __builtin_bit_cast(unsigned int, m);
  const unsigned int x = w ^ (mu | 0x80008000u);
  const u16x2 c = __builtin_bit_cast(u16x2, mu) + (u16x2){0x80, 0x80};
  u16x2 k = __builtin_bit_cast(u16x2, x) - c;
  k = __builtin_elementwise_min(k, (u16x2){0xFF01, 0xFF01});
  return __builtin_bit_cast(unsigned int, k);
}

// 32-bit order key of a float32 with the same conventions.
__device__ inline unsigned int f32_key(unsigned int b) {
  const unsigned int m = (unsigned int)((int)b >> 31);
  const unsigned int x = b ^ (m | 0x80000000u);
  const unsigned int k = x - (m + 0x00800000u);
  return k < 0xFF000001u ? k : 0xFF000001u;
}

// Partial of a unit: key in the high word, 0xFFFFFFFF - index in the low word,
// so the maximum is the largest value at the lowest index. 0 = no element.
__device__ inline unsigned long long pack_best(unsigned int key, unsigned int gidx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - gidx);
}

template <typename T>
__device__ inline T wave_max(T v) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const T o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

template <typename T>
__device__ inline T wave_min(T v) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const T o = __shfl_xor(v, off, kWave);
    v = o < v ? o : v;
  }
  return v;
}

// Exact per-thread (key, lowest index) over this thread's elements of a unit.
template <dspark_dtype DT>
__device__ inline unsigned long long exact_thread_best(const u32x4* d, int v0, int v1) {
  const int tid = threadIdx.x;
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
  unsigned long long best = 0;
  if constexpr (DT == DSPARK_BF16) {
    // key << 16 | (0xFFFF - p) with p = j * 8 + element: the in-thread order
    unsigned int b32 = 0;
#pragma unroll
    for (int j = 0; j < kAccVecsPerThread; ++j) {
      if (v0 + j * kAccThreads + tid < v1) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned int k = bf16x2_keys(d[j][w]);
          const unsigned int p = (unsigned int)(j * 8 + w * 2);
          const unsigned int lo = (k << 16) | (0xFFFFu - p);
          const unsigned int hi = (k & 0xFFFF0000u) | (0xFFFFu - (p + 1));
          b32 = max(b32, max(lo, hi));
        }
      }
    }
    if (b32) {
      const unsigned int p = 0xFFFFu - (b32 & 0xFFFFu);
      const unsigned int v = (unsigned int)(v0 + (int)(p >> 3) * kAccThreads + tid);
      best = pack_best(b32 >> 16, v * kEpv + (p & 7u));
    }
  } else {
    unsigned long long b64 = 0;
#pragma unroll
    for (int j = 0; j < kAccVecsPerThread; ++j) {
      if (v0 + j * kAccThreads + tid < v1) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned int p = (unsigned int)(j * 4 + w);
          const unsigned long long c =
              ((unsigned long long)f32_key(d[j][w]) << 32) | (0xFFFFFFFFu - p);
          b64 = c > b64 ? c : b64;
        }
      }
    }
    if (b64) {
      const unsigned int p = 0xFFFFFFFFu - (unsigned int)(b64 & 0xFFFFFFFFu);
      const unsigned int v = (unsigned int)(v0 + (int)(p >> 2) * kAccThreads + tid);
      best = pack_best((unsigned int)(b64 >> 32), v * kEpv + (p & 3u));
    }
  }
  return best;
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kAccThreads) void accept_argmax_kernel(AcceptArgs a) {
  __shared__ int s_max[kWaves];
  __shared__ unsigned int s_idx[kWaves];
  __shared__ unsigned long long s_best[kWaves];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int total = a.fixed_rows >= 0 ? a.fixed_rows : a.cu[a.B];
  const int total_eff = min(max(total, 0), a.max_rows);
  if (blockIdx.x == 0 && tid == 0) {
    a.meta[0] = total;
    a.meta[1] = total != total_eff ? DSPARK_DATA_BAD_LENS : 0;
  }
  const int u = blockIdx.x;
  if (u >= total_eff * a.chunks) return;
  const int row = u / a.chunks;
  const int chunk = u - row * a.chunks;
  const u32x4* rp = reinterpret_cast<const u32x4*>(a.logits + (size_t)row * a.ld_bytes);
  const int v0 = chunk * a.chunk_vecs;
  const int v1 = min(v0 + a.chunk_vecs, a.nvec);
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;

  u32x4 d[kAccVecsPerThread];
#pragma unroll
  for (int j = 0; j < kAccVecsPerThread; ++j) {
    const int v = v0 + j * kAccThreads + tid;
    // -0.0 fill: below any positive value, never a NaN
    d[j] = (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    if (v < v1) d[j] = __builtin_nontemporal_load(rp + v);
  }

  unsigned long long best = 0;
  bool exact = true;
  if constexpr (DT == DSPARK_BF16) {
    // fast path: raw signed-16 max and NaN detection
    i16x2 mi = (i16x2){(short)0x8000, (short)0x8000};
    u16x2 mu = (u16x2){0, 0};
#pragma unroll
    for (int j = 0; j < kAccVecsPerThread; ++j) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned int x = d[j][w];
        mi = __builtin_elementwise_max(mi, as_i16x2(x));
        mu = __builtin_elementwise_max(mu, as_u16x2(x));
      }
    }
    const int lm = max((int)mi[0], (int)mi[1]);
    const int lu = max((int)mu[0], (int)mu[1]);
    // positive NaN: raw value above +inf (0x7F80); negative NaN: above 0xFF80 unsigned
    int v = (lm > 0x7F80 || lu > 0xFF80) ? 0x7FFFFFFF : lm;
    v = wave_max(v);
    if (lane == 0) s_max[wave] = v;
    __syncthreads();
    int M = s_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = max(M, s_max[w]);
    if (M > 0 && M <= 0x7F80) {  // uniform over the workgroup
      exact = false;
      unsigned int cand = 0xFFFFFFFFu;
      if (lm == M) {
        // this lane holds the maximum: its first position (lowest j, w, half)
#pragma unroll
        for (int j = kAccVecsPerThread - 1; j >= 0; --j) {
#pragma unroll
          for (int w = 3; w >= 0; --w) {
            const unsigned int x = d[j][w];
            const unsigned int base = (unsigned int)(v0 + j * kAccThreads + tid) * 8u + 2u * w;
            if ((int)(short)(x >> 16) == M) cand = base + 1u;
            if ((int)(short)(x & 0xFFFFu) == M) cand = base;
          }
        }
      }
      cand = wave_min(cand);
      if (lane == 0) s_idx[wave] = cand;
      __syncthreads();
      if (tid == 0) {
        unsigned int c = s_idx[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) c = min(c, s_idx[w]);
        best = pack_best((unsigned int)M + 0x7F80u, c);
      }
    }
  }
  if (exact) {  // uniform over the workgroup
    unsigned long long b = exact_thread_best<DT>(d, v0, v1);
    b = wave_max(b);
    if (lane == 0) s_best[wave] = b;
    __syncthreads();
    if (tid == 0) {
      best = s_best[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) best = s_best[w] > best ? s_best[w] : best;
    }
  }
  if (tid == 0) {
    // elements after the last whole vector (V * size not a multiple of 16)
    if (a.tail && chunk == a.chunks - 1) {
      const unsigned char* row_p = a.logits + (size_t)row * a.ld_bytes;
      for (int t = 0; t < a.tail; ++t) {
        const unsigned int gi = (unsigned int)(a.nvec * kEpv + t);
        unsigned int key;
        if constexpr (DT == DSPARK_BF16) {
          key = bf16x2_keys((unsigned int)reinterpret_cast<const unsigned short*>(row_p)[gi]) &
                0xFFFFu;
        } else {
          key = f32_key(reinterpret_cast<const unsigned int*>(row_p)[gi]);
        }
        const unsigned long long c = pack_best(key, gi);
        best = c > best ? c : best;
      }
    }
    a.partials[u] = best;
  }
}

__device__ inline int merge_row(const AcceptArgs& a, int row) {
  const unsigned long long* p = a.partials + (size_t)row * a.chunks;
  unsigned long long m = 0;
  for (int c = 0; c < a.chunks; ++c) m = p[c] > m ? p[c] : m;
  return (int)(0xFFFFFFFFu - (unsigned int)(m & 0xFFFFFFFFu));
}

// One wave per request (blockIdx.x = r), plus a grid-stride pass that writes
// the argmax of every row. CAP = false: packed rows cu[r] .. cu[r+1]-1.
// CAP = true: strided rows r * (gamma + 1) + j, every one of them computed.
// The loads come in two rounds, each issued before anything waits on it:
// first the layout words, drafts and prefix; then every partial the wave
// needs (its row of the row pass and the request's rows). Stores follow.
template <bool CAP>
__global__ __launch_bounds__(kWave) void accept_finalize_kernel(AcceptArgs a) {
  __shared__ int am[DSPARK_MAX_GAMMA + 1];
  const int lane = threadIdx.x;
  const int G = a.gamma;
  const int r = blockIdx.x;
  const bool has_req = r < a.B;
  // round 1
  const int total = CAP ? a.fixed_rows : a.cu[a.B];
  int c0 = 0, len = 0;  // first row, verify length
  if (has_req) {
    if constexpr (CAP) {
      c0 = r * (G + 1);
      len = a.lens[r];
    } else {
      c0 = a.cu[r];
      len = a.cu[r + 1] - c0;
    }
  }
  const int dr = (has_req && lane < G) ? a.drafts[(size_t)r * G + lane] : 0;
  const int prefix = (has_req && a.prefix) ? a.prefix[r] : 0;
  const int total_eff = min(max(total, 0), a.max_rows);
  bool ok;
  if constexpr (CAP) {
    ok = len >= 1 && len <= G + 1;
  } else {
    ok = c0 >= 0 && len >= 1 && len <= G + 1 && c0 + len <= total_eff;
  }
  // round 2
  const int i0 = blockIdx.x * kWave + lane;
  const int n_rows = CAP ? G + 1 : len;  // rows whose predictions are read
  const bool need = has_req && (CAP || ok);
  const int g0 = i0 < total_eff ? merge_row(a, i0) : 0;
  const int m0 = (need && lane < n_rows) ? merge_row(a, c0 + lane) : 0;
  const int m1 = (need && lane + kWave < n_rows) ? merge_row(a, c0 + lane + kWave) : 0;
  if (i0 < total_eff) a.row_am[i0] = g0;
  for (int i = i0 + gridDim.x * kWave; i < total_eff; i += gridDim.x * kWave) {
    a.row_am[i] = merge_row(a, i);
  }
  if (!has_req) return;
  if (need) {
    if (lane < n_rows) am[lane] = m0;
    if (lane + kWave < n_rows) am[lane + kWave] = m1;
  }
  __syncthreads();
  int32_t* out = a.out_tokens + (size_t)r * (G + 1);
  // drafts compared: len - 1 of them, or all gamma for the ceiling
  const int n_chk = CAP ? G : len - 1;
  int c = 0;
  if (need) {
    // draft k (0-based, k < n_chk <= 64) against the prediction of row k
    const bool mismatch = lane < n_chk && dr != am[lane];
    const unsigned long long mm = __ballot(mismatch);
    c = mm ? (int)__builtin_ctzll(mm) : n_chk;
    if constexpr (CAP) {
      if (lane == 0) a.ceiling[r] = c;
      c = min(c, len - 1);
    }
  }
  if (!ok) {
    for (int j = lane; j <= G; j += kWave) out[j] = -1;
    if (a.mask) {
      for (int k = lane; k < G; k += kWave) a.mask[(size_t)r * G + k] = 0;
    }
    if (lane == 0) {
      a.num_correct[r] = 0;
      a.bonus[r] = -1;
      a.commit[r] = 0;
      if (a.new_seq) a.new_seq[r] = prefix;
      atomicOr(a.meta + 1, DSPARK_DATA_BAD_LENS);
    }
    return;
  }
  const int bon = am[c];
  // column j < gamma holds draft j (lane j's register); column gamma starts at -1
  for (int j = lane; j <= G; j += kWave) out[j] = j == c ? bon : (j < G ? dr : -1);
  if (a.mask) {
    for (int k = lane; k < G; k += kWave) a.mask[(size_t)r * G + k] = k < c ? 1 : 0;
  }
  if (lane == 0) {
    a.num_correct[r] = c;
    a.bonus[r] = bon;
    a.commit[r] = c + 1;
    if (a.new_seq) a.new_seq[r] = prefix + c + 1;
  }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, dspark_dtype dt, int grid, hipStream_t s) {
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(accept_argmax_kernel<DSPARK_BF16>, dim3(grid), dim3(kAccThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(accept_argmax_kernel<DSPARK_F32>, dim3(grid), dim3(kAccThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fgrid = a.B > 0 ? a.B : 1;
  if (a.fixed_rows >= 0) {
    hipLaunchKernelGGL(accept_finalize_kernel<true>, dim3(fgrid), dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL(accept_finalize_kernel<false>, dim3(fgrid), dim3(kWave), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
