// Internal declarations shared by the HIP kernels of libdspark (gfx950 only).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;

// ---------------------------------------------------------------- kernels

struct PlanArgs {
  int B, gamma, kind, lmin, lmax, b_lo, b_hi, theta_len;
  int cost_mode;  // dspark_cost_mode
  int sps_len;
  int align;      // graph-tier alignment (fused plan + pack only)
  const int32_t* sps_m;
  const float* sps;
  float eps, bias;
  const float* conf;
  const float* temps;
  const float* alpha;
  const float* theta;
  int32_t* lens;
  int32_t* meta;
  double* val;
  float* surv_out;
  double* sweep;
};
constexpr int kPlanThreads = 1024;
size_t plan_lds_bytes(int B, int gamma, int n_keys);

struct PackArgs {
  int B, gamma, ntiers;
  const int32_t* lens;
  const int32_t* anchors;
  const int32_t* drafts;
  const int32_t* prefix;
  int32_t* cu;
  int32_t* ids;
  int32_t* req;
  int32_t* pos;
  int32_t* meta;
  int32_t tiers[DSPARK_MAX_TIERS];
};
constexpr int kPackThreads = 1024;
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
// plan, then (p != nullptr) pack in the same workgroup
hipError_t launch_plan(const PlanArgs& a, const PackArgs* p, hipStream_t s);

struct AcceptArgs {
  const unsigned char* logits;
  int64_t ld_bytes;
  int V, max_rows, B, gamma;
  // -1: packed rows described by cu; >= 0: the strided layout of cap-accept,
  // B * (gamma + 1) rows, request r at rows r * (gamma + 1) + j
  int fixed_rows;
  int chunks;      // units per row
  int chunk_vecs;  // 16-byte vectors per unit
  int nvec;        // whole 16-byte vectors per row
  int tail;        // elements after the last whole vector
  const int32_t* cu;
  const int32_t* drafts;
  const int32_t* prefix;
  int32_t* row_am;
  int32_t* num_correct;
  int32_t* bonus;
  int32_t* commit;
  int32_t* out_tokens;
  int32_t* new_seq;
  uint8_t* mask;
  int32_t* meta;
  unsigned long long* partials;  // [max_rows * chunks] (key, index) per unit
  const int32_t* lens;  // cap-accept: verify_lens [B]
  int32_t* ceiling;     // cap-accept: uncapped leading matches [B]
};
constexpr int kAccThreads = 256;
constexpr int kAccVecsPerThread = 8;
constexpr int kAccMaxChunkVecs = kAccThreads * kAccVecsPerThread;
hipError_t launch_accept(const AcceptArgs& a, dspark_dtype dt, int grid, hipStream_t s);

struct ScatterArgs {
  const unsigned char* src;
  int64_t src_ld;  // bytes
  unsigned char* dst;
  int64_t dst_ld;  // bytes
  int B, stride, max_rows;
  int chunks;      // units per row
  int chunk_vecs;  // 16-byte vectors per unit
  int nvec;        // whole 16-byte vectors per row
  int tail;        // bytes after the last whole vector
  const int32_t* cu;
  int32_t* meta;
};
constexpr int kScatterThreads = 256;
constexpr int kScatterVecsPerThread = 2;
constexpr int kScatterRows = 8;  // rows of a request copied per batch
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s);

struct TvArgs {
  const unsigned char* q;
  int64_t ldq_bytes;
  const unsigned char* p;
  int64_t ldp_bytes;
  int V, B, gamma, rows_per_req;
  int nvec, tail;
  float* a_out;
  float* s_out;
};
constexpr int kTvThreads = 1024;
hipError_t launch_tv(const TvArgs& a, dspark_dtype dt, hipStream_t s);

struct StsArgs {
  int N, gamma, n_t, nbins;
  int per_block, n_blocks;  // records per workgroup of the bin kernel, workgroups
  const float* z;           // [N, gamma] confidence logits
  const uint8_t* labels;    // [N, gamma] greedy prefix labels (nonzero = survived)
  float grid[DSPARK_STS_MAX_GRID];
  float* temps;             // [gamma]
  int32_t* t_index;         // [gamma]
  double* ece;              // [gamma]
  double* brier;            // [gamma]
  double* ece_grid;         // [gamma, n_t] or null
  float* surv_out;          // [N, gamma] or null
  float* s_work[2];         // workspace: two [N] survival buffers, used alternately
  long long* hists;         // workspace: [3][n_t][2 * nbins + 1] summed histograms,
                            // position k in buffer k % 3
};
constexpr int kStsPass = 256;        // records a bin workgroup takes at a time
constexpr int kStsPhases = 4;        // threads per record, each on every 4th candidate
constexpr int kStsBinThreads = kStsPass * kStsPhases;
constexpr int kStsThreads = 256;     // finish and clear kernels
constexpr int kStsMaxBlocks = 1024;  // bin workgroups at most
hipError_t launch_sts(const StsArgs& a, hipStream_t s);

// Chain speculative-sampling accept (sampling.hip).
struct SampJob {
  int mode;  // 0 none, 1 draw from p, 2 draw from the residual of (p, q)
  int prow, qrow;
  unsigned int word;
  int col;  // output column of the drawn token (= num_correct)
  float mp, mq;  // row maxima
  int pad;
  unsigned long long zp, zq;  // weight sums
};
struct SampArgs {
  const unsigned char* tgt;  // packed target rows
  int64_t ld_t;              // bytes
  const unsigned char* drf;  // draft rows, row r * gamma + k - 1 for draft k
  int64_t ld_q;              // bytes
  int V, nvec, tail, chunks, chunk_vecs, max_rows, B, gamma;
  const int32_t* cu;
  const int32_t* drafts;
  const float* temps;
  const uint32_t* ra;  // [B, gamma]
  const uint32_t* rs;  // [B, gamma + 1]
  const int32_t* prefix;
  int32_t* num_correct;
  int32_t* bonus;
  int32_t* commit;
  int32_t* out_tokens;
  int32_t* new_seq;
  int32_t* meta;
  // workspace, per slot and chunk: target slots r * (gamma + 1) + j (packed
  // row cu[r] + j), then draft slots B * (gamma + 1) + r * gamma + k (draft
  // row r * gamma + k)
  int rowstat;                // the row statistics come from samp_rowstat_kernel
  unsigned long long* kpart;  // maximum key with its index
  unsigned long long* zpart;  // weight sum
  unsigned long long* rpart;  // [B, chunks, kRsumParts, 2]: residual member sums of Wp, Wq
  SampJob* jobs;              // [B]
};
constexpr int kSampThreads = 256;       // max and weight-sum kernels
constexpr int kSampVecsPerThread = 8;
constexpr int kSampChunkVecs = kSampThreads * kSampVecsPerThread;
constexpr int kSampDrawThreads = 1024;  // draw kernel
constexpr int kRsumParts = 2;           // residual-sum workgroups per chunk
constexpr int kSampMaxChunks = 32;      // chunks of a DSPARK_MAX_VOCAB float32 row
constexpr int kRsThreads = 1024;        // row-statistics kernel
constexpr int kRsMaxSlots = 16;         // 16-byte register slots per thread, at most
constexpr int kRsMaxList = 64;          // rows per row-statistics workgroup, at most
hipError_t launch_sampling(const SampArgs& a, dspark_dtype dt, hipStream_t s);

// Compute units of the current device, queried once per device (the
// persistent kernels launch one workgroup per CU).
hipError_t current_cu_count(int* cus);

// ---------------------------------------------------------------- helpers

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ inline T wave_sum(T v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// n / d for 0 <= n < 2^15 and 1 <= d <= 65 with one float32 multiply and a
// truncation, exact: with inv = RN32((1 + 2^-22) / d) = (1 + e) / d,
// e in [2^-22 - 2^-23.9, 2^-22 + 2^-23.9], and n = q d + f (0 <= f < d), the
// product RN32(n * inv) = (n / d)(1 + e)(1 + h), |h| <= 2^-24, is at least
// n / d >= q and at most n / d + (n / d) 2^-21 < q + (d - 1) / d + 2^-6 / d
// < q + 1, so it truncates to q.
struct SmallDiv {
  float inv;
  int d;
  __device__ explicit SmallDiv(int d_) : inv(__fdiv_rn(1.0f + 0x1p-22f, (float)d_)), d(d_) {}
  __device__ int quo(int n) const { return (int)__fmul_rn((float)n, inv); }
};

// ---- wave primitives on DPP (data-parallel primitives): lane exchanges
// inside the VALU, no LDS round trip. Encodings of the gfx9-family DPP
// controls used here: row_shr:n = 0x110 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143. A lane whose source lies outside its 16-lane row,
// or whose row is masked off, receives `ident`.

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline uint32_t dpp32(uint32_t x, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline uint64_t dpp64(uint64_t x, uint64_t ident) {
  const uint32_t lo = dpp32<CTRL, ROW_MASK>((uint32_t)x, (uint32_t)ident);
  const uint32_t hi = dpp32<CTRL, ROW_MASK>((uint32_t)(x >> 32), (uint32_t)(ident >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK = 0xF, typename T>
__device__ inline T dpp_t(T x, T ident) {
  if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, dpp64<CTRL, ROW_MASK>(__builtin_bit_cast(uint64_t, x),
                                                       __builtin_bit_cast(uint64_t, ident)));
  } else {
    return __builtin_bit_cast(T, dpp32<CTRL, ROW_MASK>(__builtin_bit_cast(uint32_t, x),
                                                       __builtin_bit_cast(uint32_t, ident)));
  }
}

// Inclusive scan over the 64 lanes of a wave for an associative `op` with
// identity `ident` (Hillis-Steele inside each 16-lane row, then the row
// totals carried to the later rows).
template <typename T, typename Op>
__device__ inline T wave_incl_scan_op(T x, T ident, Op op) {
  x = op(x, dpp_t<0x111>(x, ident));
  x = op(x, dpp_t<0x112>(x, ident));
  x = op(x, dpp_t<0x114>(x, ident));
  x = op(x, dpp_t<0x118>(x, ident));
  x = op(x, dpp_t<0x142, 0xA>(x, ident));
  x = op(x, dpp_t<0x143, 0xC>(x, ident));
  return x;
}

template <typename T>
__device__ inline T read_lane(T x, int lane) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
  }
}

struct OpAdd {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};

// Inclusive scan inside each 16-lane row.
template <typename T, typename Op>
__device__ inline T row_incl_scan(T x, T ident, Op op) {
  x = op(x, dpp_t<0x111>(x, ident));
  x = op(x, dpp_t<0x112>(x, ident));
  x = op(x, dpp_t<0x114>(x, ident));
  x = op(x, dpp_t<0x118>(x, ident));
  return x;
}

// Exclusive scan over the block, without a closing barrier: for callers that
// pass another barrier before anything writes `wsum` (one slot per wave)
// again. Returns the exclusive prefix of this thread's value; *total receives
// the block total. With 16 waves and integer sums, every 16-lane row reads all
// 16 wave totals (lane l takes wave l & 15's) and scans them with four row
// shifts.
template <typename T, int NTHREADS>
__device__ inline T block_excl_scan_open(T v, T* wsum, T* total) {
  constexpr int kWaves = NTHREADS / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const T incl = wave_incl_scan_op(v, T(0), OpAdd{});
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if constexpr (kWaves == 16 && std::is_integral_v<T>) {
    const T t = row_incl_scan(wsum[lane & 15], T(0), OpAdd{});
    *total = read_lane(t, 15);
    return (wave > 0 ? read_lane(t, wave - 1) : T(0)) + incl - v;
  } else {
    const T t = lane < kWaves ? wsum[lane] : T(0);
    const T tincl = wave_incl_scan_op(t, T(0), OpAdd{});
    *total = read_lane(tincl, kWaves - 1);
    return (wave > 0 ? read_lane(tincl, wave - 1) : T(0)) + incl - v;
  }
}

// Exclusive scan over the block (block_excl_scan_open, then a barrier so that
// `wsum` may be reused right after).
template <typename T, int NTHREADS>
__device__ inline T block_excl_scan(T v, T* wsum, T* total) {
  const T r = block_excl_scan_open<T, NTHREADS>(v, wsum, total);
  __syncthreads();
  return r;
}

// Reduction over the block with `op` (identity `ident`), result in every
// thread. `wsum` needs one slot per wave.
template <typename T, int NTHREADS, typename Op>
__device__ inline T block_reduce(T v, T ident, Op op, T* wsum) {
  constexpr int kWaves = NTHREADS / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  v = wave_incl_scan_op(v, ident, op);
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  T t = lane < kWaves ? wsum[lane] : ident;
  t = read_lane(wave_incl_scan_op(t, ident, op), kWave - 1);
  __syncthreads();
  return t;
}

template <typename T, int NTHREADS>
__device__ inline T block_sum(T v, T* wsum) {
  return block_reduce<T, NTHREADS>(v, T(0), OpAdd{}, wsum);
}

}  // namespace dspark
