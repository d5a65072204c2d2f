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
// The vocabulary pass is a pure stream of total*V elements (about 596 MB at
// 2304 rows x 129280 bf16) read once, so the kernel is built for HBM
// bandwidth, not for matrix cores:
//   * a persistent grid of 256-thread workgroups walks (row, chunk) units of
//     up to 2048 16-byte vectors (32 KB); eight vectors per thread are in
//     flight per unit, and eight resident workgroups per CU keep about
//     256 KB of loads outstanding per CU;
//   * loads are 16-byte nontemporal (the logits are read exactly once);
//   * bf16 elements become 16-bit order keys with packed 16-bit integer ops
//     (two elements per instruction). NaN maps to the top, -0 and +0 to the
//     same key. Each key carries its in-thread position in the low half of a
//     32-bit word, so one v_max3_u32 folds two elements into the running
//     (value, lowest index) maximum;
//   * a unit's maximum goes to a workspace slot. The last unit of a row
//     (atomic counter) merges the row; the last row overall finalizes every
//     request. No workgroup ever waits for another, and the counters return
//     to zero before the kernel ends.
#include "common.h"

namespace dspark {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// 16-bit order key of two bf16 values packed in one dword (each half
// independently): larger value -> larger key; -0 == +0; NaN above +inf.
//   m = sign mask (0xFFFF for negatives); key = (h ^ (m | 0x8000)) - m maps
//   the sign-magnitude bits to an order-preserving integer (-0 and +0 both to
//   0x8000, -inf to 0x0080). Subtracting 0x80 moves -inf to 0 and every NaN to
//   0xFF01..0xFFFF (wrapping), and the final min folds all NaNs onto 0xFF01.
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

__device__ inline unsigned long long pack_best(unsigned int key, unsigned int gidx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - gidx);
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Best (key, lowest index) of one unit for this thread, as a packed u64
// (0 if the thread owns no element of the unit).
template <dspark_dtype DT>
__device__ inline unsigned long long unit_scan(const AcceptArgs& a, int row, int chunk) {
  const int tid = threadIdx.x;
  const u32x4* rp = reinterpret_cast<const u32x4*>(a.logits + (size_t)row * a.ld_bytes);
  const int v0 = chunk * a.chunk_vecs;
  const int v1 = min(v0 + a.chunk_vecs, a.nvec);
  u32x4 d[kAccVecsPerThread];
#pragma unroll
  for (int j = 0; j < kAccVecsPerThread; ++j) {
    const int v = v0 + j * kAccThreads + tid;
    if (v < v1) d[j] = __builtin_nontemporal_load(rp + v);
  }
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;  // elements per 16-byte vector
  unsigned long long best = 0;
  if constexpr (DT == DSPARK_BF16) {
    // packed: key << 16 | (0xFFFF - p), p = j * 8 + element (in-thread order)
    const unsigned int hi_mask = 0xFFFF0000u;
    unsigned int b32 = 0;
#pragma unroll
    for (int j = 0; j < kAccVecsPerThread; ++j) {
      if (v0 + j * kAccThreads + tid < v1) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned int k = bf16x2_keys(d[j][w]);
          const unsigned int p = (unsigned int)(j * 8 + w * 2);
          const unsigned int lo = (k << 16) | (0xFFFFu - p);
          const unsigned int hi = (k & hi_mask) | (0xFFFFu - (p + 1));
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
  // elements after the last whole vector (V * size not a multiple of 16)
  if (a.tail && chunk == a.chunks - 1 && tid == 0) {
    const unsigned char* row_p = a.logits + (size_t)row * a.ld_bytes;
    for (int t = 0; t < a.tail; ++t) {
      const unsigned int gi = (unsigned int)(a.nvec * kEpv + t);
      unsigned int key;
      if constexpr (DT == DSPARK_BF16) {
        const unsigned short h = reinterpret_cast<const unsigned short*>(row_p)[gi];
        key = bf16x2_keys((unsigned int)h) & 0xFFFFu;
      } else {
        key = f32_key(reinterpret_cast<const unsigned int*>(row_p)[gi]);
      }
      const unsigned long long c = pack_best(key, gi);
      best = c > best ? c : best;
    }
  }
  return best;
}

__device__ inline int load_am(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Finalize every request (one workgroup). Row argmaxes come from other
// workgroups, so they are read with agent-scope atomic loads after an
// acquire fence.
__device__ void finalize(const AcceptArgs& a, int total, int total_eff) {
  __shared__ int s_status;
  const int tid = threadIdx.x;
  if (tid == 0) s_status = total != total_eff ? DSPARK_DATA_BAD_LENS : 0;
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int G = a.gamma;
  int bad = 0;
  for (int r = tid; r < a.B; r += kAccThreads) {
    const int c0 = a.cu[r], c1 = a.cu[r + 1];
    const int len = c1 - c0;
    const int prefix = a.prefix ? a.prefix[r] : 0;
    const int32_t* dr = a.drafts + (size_t)r * G;
    int32_t* out = a.out_tokens + (size_t)r * (G + 1);
    if (!(c0 >= 0 && len >= 1 && len <= G + 1 && c1 <= total_eff)) {
      bad = 1;
      a.num_correct[r] = 0;
      a.bonus[r] = -1;
      a.commit[r] = 0;
      if (a.new_seq) a.new_seq[r] = prefix;
      for (int j = 0; j <= G; ++j) out[j] = -1;
      if (a.mask) {
        for (int k = 0; k < G; ++k) a.mask[(size_t)r * G + k] = 0;
      }
      continue;
    }
    int c = 0;
    bool run = true;
    for (int k = 0; k < len - 1; ++k) {
      const bool m = dr[k] == load_am(a.row_am + c0 + k);
      run = run && m;
      c += run ? 1 : 0;
    }
    const int bon = load_am(a.row_am + c0 + c);
    a.num_correct[r] = c;
    a.bonus[r] = bon;
    a.commit[r] = c + 1;
    if (a.new_seq) a.new_seq[r] = prefix + c + 1;
    for (int j = 0; j < G; ++j) out[j] = j == c ? bon : dr[j];
    out[G] = c == G ? bon : -1;
    if (a.mask) {
      for (int k = 0; k < G; ++k) a.mask[(size_t)r * G + k] = k < c ? 1 : 0;
    }
  }
  if (bad) atomicOr(&s_status, DSPARK_DATA_BAD_LENS);
  __syncthreads();
  if (tid == 0) {
    a.meta[0] = total;
    a.meta[1] = s_status;
  }
}

template <dspark_dtype DT>
__global__ __launch_bounds__(kAccThreads) void accept_kernel(AcceptArgs a) {
  __shared__ unsigned long long s_best[2][kAccThreads / kWave];
  __shared__ int s_final;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

  const int total = a.cu[a.B];
  const int total_eff = min(max(total, 0), a.max_rows);
  const int units = total_eff * a.chunks;
  bool is_final = false;
  int par = 0;
  for (int u = blockIdx.x; u < units; u += gridDim.x, par ^= 1) {
    const int row = u / a.chunks;
    const int chunk = u - row * a.chunks;
    unsigned long long best = unit_scan<DT>(a, row, chunk);
    best = wave_max_u64(best);
    if (lane == 0) s_best[par][wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long m = s_best[par][0];
      for (int w = 1; w < kAccThreads / kWave; ++w) m = s_best[par][w] > m ? s_best[par][w] : m;
      a.partials[u] = m;
      const unsigned int old = __hip_atomic_fetch_add(a.row_cnt + row, 1u, __ATOMIC_RELEASE,
                                                      __HIP_MEMORY_SCOPE_AGENT);
      if (old == (unsigned int)(a.chunks - 1)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        unsigned long long rm = 0;
        for (int c = 0; c < a.chunks; ++c) {
          const unsigned long long pc = __hip_atomic_load(
              a.partials + (size_t)row * a.chunks + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          rm = pc > rm ? pc : rm;
        }
        a.row_am[row] = (int32_t)(0xFFFFFFFFu - (unsigned int)(rm & 0xFFFFFFFFu));
        __hip_atomic_store(a.row_cnt + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned int done = __hip_atomic_fetch_add(a.glob_cnt, 1u, __ATOMIC_ACQ_REL,
                                                         __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned int)(total_eff - 1)) {
          __hip_atomic_store(a.glob_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          is_final = true;
        }
      }
    }
  }
  // The finalizing workgroup is the one that completed the last row; with no
  // rows at all, workgroup 0 finalizes.
  if (tid == 0) s_final = (is_final || (units == 0 && blockIdx.x == 0)) ? 1 : 0;
  __syncthreads();
  if (s_final) finalize(a, total, total_eff);
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, dspark_dtype dt, int grid, hipStream_t s) {
  if (dt == DSPARK_BF16) {
    hipLaunchKernelGGL(accept_kernel<DSPARK_BF16>, dim3(grid), dim3(kAccThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(accept_kernel<DSPARK_F32>, dim3(grid), dim3(kAccThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
