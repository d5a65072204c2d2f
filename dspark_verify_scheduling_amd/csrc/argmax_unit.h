// Per-unit argmax over a row's 16-byte vectors, shared by the greedy accept
// (accept.hip) and the sampling accept (sampling.hip).
//
// A unit is up to kAccThreads * kAccVecsPerThread vectors of one row, loaded
// by the caller into d[] (vector v0 + j * kAccThreads + tid in d[j]; lanes
// past v1 hold the -0.0 fill). The result, valid in thread 0, is the 64-bit
// partial key << 32 | (0xFFFFFFFF - index): the largest value at the lowest
// index. Values compare as float32 after exact bfloat16 widening, -0 == +0
// and NaN ranks above every number. Keys are 16-bit for bfloat16 (see
// bf16x2_keys) and 32-bit for float32 (see f32_key); best_value and best_bad
// decode them.
#pragma once

#include "common.h"

namespace dspark {
namespace argmax {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kUnitWaves = kAccThreads / kWave;

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


struct UnitSmem {
  int max[kUnitWaves];
  unsigned int idx[kUnitWaves];
  unsigned long long best[kUnitWaves];
};

template <dspark_dtype DT>
__device__ inline unsigned long long unit_best(const u32x4* d, int v0, int v1,
                                               const unsigned char* row_p, int nvec, int tail,
                                               bool last_chunk, UnitSmem& sm) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  constexpr int kEpv = DT == DSPARK_BF16 ? 8 : 4;
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
    if (lane == 0) sm.max[wave] = v;
    __syncthreads();
    int M = sm.max[0];
#pragma unroll
    for (int w = 1; w < kUnitWaves; ++w) M = max(M, sm.max[w]);
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
      if (lane == 0) sm.idx[wave] = cand;
      __syncthreads();
      if (tid == 0) {
        unsigned int c = sm.idx[0];
#pragma unroll
        for (int w = 1; w < kUnitWaves; ++w) c = min(c, sm.idx[w]);
        best = pack_best((unsigned int)M + 0x7F80u, c);
      }
    }
  }
  if (exact) {  // uniform over the workgroup
    unsigned long long b = exact_thread_best<DT>(d, v0, v1);
    b = wave_max(b);
    if (lane == 0) sm.best[wave] = b;
    __syncthreads();
    if (tid == 0) {
      best = sm.best[0];
#pragma unroll
      for (int w = 1; w < kUnitWaves; ++w) best = sm.best[w] > best ? sm.best[w] : best;
    }
  }
  if (tid == 0) {
    // elements after the last whole vector (V * size not a multiple of 16)
    if (tail && last_chunk) {
      for (int t = 0; t < tail; ++t) {
        const unsigned int gi = (unsigned int)(nvec * kEpv + t);
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
  }
  return best;
}

// The maximum value of a partial (both zeros decode to +0); meaningful when
// best_bad is false.
template <dspark_dtype DT>
__device__ inline float best_value(unsigned long long b) {
  const unsigned int k = (unsigned int)(b >> 32);
  if constexpr (DT == DSPARK_BF16) {
    const unsigned int h = k >= 0x7F80u ? k - 0x7F80u : (~(k + 0x7Fu) & 0xFFFFu);
    return __uint_as_float(h << 16);
  } else {
    return __uint_as_float(k >= 0x7F800000u ? k - 0x7F800000u : ~(k + 0x007FFFFFu));
  }
}

// NaN or +inf maximum (a NaN anywhere ranks highest), or -inf (no finite
// element), or no element at all.
template <dspark_dtype DT>
__device__ inline bool best_bad(unsigned long long b) {
  const unsigned int k = (unsigned int)(b >> 32);
  if (b == 0) return true;
  if constexpr (DT == DSPARK_BF16) {
    return k >= 0xFF00u || k == 0u;
  } else {
    return k >= 0xFF000000u || k == 0u;
  }
}

__device__ inline int best_index(unsigned long long b) {
  return (int)(0xFFFFFFFFu - (unsigned int)b);
}

}  // namespace argmax
}  // namespace dspark
