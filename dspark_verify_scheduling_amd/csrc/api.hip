// C ABI of libdspark: argument validation on the host, then kernel launches
// on the caller's stream. No allocation, no synchronization, no host reads of
// device data.
#include <float.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "common.h"

namespace {

thread_local char g_last_error[512] = "";

dspark_status fail(dspark_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

dspark_status ok() {
  g_last_error[0] = '\0';
  return DSPARK_OK;
}

dspark_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    return fail(DSPARK_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  }
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(dspark_dtype dt) { return dt == DSPARK_BF16 ? 2 : 4; }

// Row geometry of the vocabulary pass: whole 16-byte vectors, tail elements,
// units (chunks) per row and vectors per unit.
struct RowGeom {
  int nvec, tail, chunks, chunk_vecs;
};

RowGeom row_geom(int V, dspark_dtype dt) {
  const int epv = (int)(16 / elem_size(dt));
  RowGeom g;
  g.nvec = V / epv;
  g.tail = V - g.nvec * epv;
  g.chunks = (g.nvec + dspark::kAccMaxChunkVecs - 1) / dspark::kAccMaxChunkVecs;
  if (g.chunks < 1) g.chunks = 1;
  g.chunk_vecs = (g.nvec + g.chunks - 1) / g.chunks;
  return g;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of dspark_sts_fit: two survival buffers, per-candidate error sums,
// per-workgroup histograms.
struct StsGeom {
  int per_block, n_blocks;
  size_t s_off[2], h_off, bytes;
};

StsGeom sts_geom(int N, int n_t, int n_bins) {
  StsGeom g;
  // whole passes of kStsPass records per workgroup, at most kStsMaxBlocks
  // workgroups
  const int want = (N + dspark::kStsMaxBlocks - 1) / dspark::kStsMaxBlocks;
  g.per_block = std::max(1, (want + dspark::kStsPass - 1) / dspark::kStsPass) * dspark::kStsPass;
  g.n_blocks = N > 0 ? (N + g.per_block - 1) / g.per_block : 1;
  const size_t sv = align256((size_t)N * sizeof(float));
  g.s_off[0] = 0;
  g.s_off[1] = sv;
  g.h_off = 2 * sv;  // three summed-histogram buffers
  g.bytes = g.h_off + align256((size_t)3 * n_t * (2 * n_bins + 1) * sizeof(long long));
  return g;
}

// Workspace of dspark_accept_sampling: a maximum key and a weight sum per
// (slot, chunk), slots B * (2 * gamma + 1); two residual sums per (request,
// chunk, part of the chunk); one draw job per request.
struct SampGeom {
  int chunks, chunk_vecs;
  size_t part_bytes, rpart_bytes, bytes;
};

SampGeom samp_geom(int B, int gamma, int V, dspark_dtype dt) {
  const RowGeom rg = row_geom(V, dt);
  SampGeom g;
  g.chunks = (rg.nvec + dspark::kSampChunkVecs - 1) / dspark::kSampChunkVecs;
  if (g.chunks < 1) g.chunks = 1;
  // whole chunks of kSampChunkVecs vectors (the last one partial): the
  // row-statistics kernel holds chunk c in its register slots 2c and 2c + 1
  g.chunk_vecs = dspark::kSampChunkVecs;
  static_assert((DSPARK_MAX_VOCAB * 4 / 16 + dspark::kSampChunkVecs - 1) / dspark::kSampChunkVecs <=
                    dspark::kSampMaxChunks,
                "the draw kernel holds the chunk sums of the longest row in LDS");
  g.part_bytes = align256((size_t)B * (2 * gamma + 1) * g.chunks * sizeof(unsigned long long));
  g.rpart_bytes =
      align256((size_t)B * g.chunks * dspark::kRsumParts * 2 * sizeof(unsigned long long));
  g.bytes = 2 * g.part_bytes + g.rpart_bytes +
            align256((size_t)(B > 0 ? B : 1) * sizeof(dspark::SampJob));
  return g;
}

// Workspace of dspark_accept: one 64-bit (key, index) partial per unit.
size_t ws_bytes(int max_rows, int chunks) {
  const size_t b = align256((size_t)max_rows * chunks * sizeof(unsigned long long));
  return b > 256 ? b : 256;
}

// The partials of dspark_accept_noalloc: a device array the library holds on
// every GPU it runs on until the process ends, so that call allocates nothing.
// In host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // threads that race here store the same address
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

namespace dspark {

hipError_t current_cu_count(int* cus) {
  // per device, 0 until queried; threads that race on the first query store
  // the same value, through atomics so that the race is well defined
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) {
      *cus = n;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}

}  // namespace dspark

extern "C" {

int32_t dspark_version(void) { return (1 << 16) | 2; }

const char* dspark_status_str(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_E_INVALID: return "DSPARK_E_INVALID";
    case DSPARK_E_UNSUPPORTED: return "DSPARK_E_UNSUPPORTED";
    case DSPARK_E_WORKSPACE: return "DSPARK_E_WORKSPACE";
    case DSPARK_E_LAUNCH: return "DSPARK_E_LAUNCH";
  }
  return "DSPARK_E_UNKNOWN";
}

const char* dspark_last_error(void) { return g_last_error; }

}  // extern "C"

// Validation shared by dspark_plan and dspark_plan_pack; fills `a`.
static dspark_status check_plan(const char* fn, int32_t B, int32_t gamma, dspark_input kind,
                                const float* conf, const float* sts_temp, int32_t min_verify_len,
                                int32_t max_verify_len, float survival_eps, int32_t budget_lo,
                                int32_t budget_hi, float cost_bias, const float* cost_alpha,
                                int32_t alpha_len, const float* cost_theta, int32_t theta_len,
                                int32_t* verify_lens, int32_t* plan_meta, double* plan_val,
                                float* survival_out, double* sweep_out, dspark::PlanArgs* a,
                                const dspark_plan_options* opt = nullptr) {
  const bool sps1d = opt && opt->cost_mode == DSPARK_COST_SPS1D;
  if (opt && opt->cost_mode != DSPARK_COST_ADDITIVE && !sps1d)
    return fail(DSPARK_E_INVALID, "%s: unknown cost mode %d", fn, (int)opt->cost_mode);
  if (sps1d && (!opt->sps_m || !opt->sps || opt->sps_len < 1 ||
                opt->sps_len > DSPARK_MAX_SPS_PROBES))
    return fail(DSPARK_E_INVALID, "%s: SPS table needs 1..%d probes and both arrays", fn,
                DSPARK_MAX_SPS_PROBES);
  if (B < 0) return fail(DSPARK_E_INVALID, "%s: B = %d < 0", fn, B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "%s: gamma = %d outside [1, %d]", fn, gamma, DSPARK_MAX_GAMMA);
  if (kind != DSPARK_IN_CONF_LOGITS && kind != DSPARK_IN_COND && kind != DSPARK_IN_SURVIVAL)
    return fail(DSPARK_E_INVALID, "%s: unknown input kind %d", fn, (int)kind);
  if (B > DSPARK_MAX_BATCH || (int64_t)B * gamma > DSPARK_MAX_CANDIDATES)
    return fail(DSPARK_E_UNSUPPORTED, "%s: B * gamma = %lld exceeds %d", fn, (long long)B * gamma,
                DSPARK_MAX_CANDIDATES);
  if (B > 0 && !conf) return fail(DSPARK_E_INVALID, "%s: conf is NULL", fn);
  if (kind == DSPARK_IN_CONF_LOGITS && !sts_temp)
    return fail(DSPARK_E_INVALID, "%s: sts_temp is NULL for confidence logits", fn);
  if (!sps1d && (!cost_alpha || !cost_theta))
    return fail(DSPARK_E_INVALID, "%s: cost table pointer is NULL", fn);
  if (!plan_meta || !plan_val || (B > 0 && !verify_lens))
    return fail(DSPARK_E_INVALID, "%s: an output pointer is NULL", fn);
  if (budget_lo < 0) return fail(DSPARK_E_INVALID, "%s: budget_lo = %d < 0", fn, budget_lo);
  if (budget_hi >= 0 && budget_lo > budget_hi)
    return fail(DSPARK_E_INVALID, "%s: budget_lo %d > budget_hi %d", fn, budget_lo, budget_hi);
  if (survival_eps != survival_eps) return fail(DSPARK_E_INVALID, "%s: survival_eps is NaN", fn);
  const int lmin = std::min(std::max(min_verify_len, 1), gamma + 1);
  const int lmax = std::min(std::max(max_verify_len, lmin), gamma + 1);
  if (!sps1d && alpha_len <= B)
    return fail(DSPARK_E_INVALID, "%s: alpha_len %d must exceed B = %d", fn, alpha_len, B);
  if (!sps1d && (int64_t)theta_len <= (int64_t)B * lmax)
    return fail(DSPARK_E_INVALID, "%s: theta_len %d must exceed B * L_max = %lld", fn, theta_len,
                (long long)B * lmax);
  a->B = B;
  a->gamma = gamma;
  a->kind = (int)kind;
  a->lmin = lmin;
  a->lmax = lmax;
  a->b_lo = budget_lo;
  a->b_hi = budget_hi < 0 ? -1 : budget_hi;
  a->theta_len = theta_len;
  a->eps = survival_eps;
  a->bias = cost_bias;
  a->conf = conf;
  a->temps = sts_temp;
  a->alpha = cost_alpha;
  a->theta = cost_theta;
  a->lens = verify_lens;
  a->meta = plan_meta;
  a->val = plan_val;
  a->surv_out = survival_out;
  a->sweep = sweep_out;
  a->cost_mode = sps1d ? DSPARK_COST_SPS1D : DSPARK_COST_ADDITIVE;
  a->sps_m = sps1d ? opt->sps_m : nullptr;
  a->sps = sps1d ? opt->sps : nullptr;
  a->sps_len = sps1d ? opt->sps_len : 0;
  a->align = (opt && opt->align_to_tier) ? 1 : 0;
  return DSPARK_OK;
}

// Validation shared by dspark_pack and dspark_plan_pack; fills `a`.
static dspark_status check_pack(const char* fn, int32_t B, int32_t gamma,
                                const int32_t* verify_lens, bool need_lens,
                                const int32_t* anchor_ids, const int32_t* draft_tokens,
                                const int32_t* tiers_host, int32_t num_tiers,
                                const int32_t* prefix_lens, int32_t* cu_seqlens,
                                int32_t* packed_ids, int32_t* packed_req, int32_t* packed_pos,
                                int32_t* pack_meta, dspark::PackArgs* a) {
  if (B < 0) return fail(DSPARK_E_INVALID, "%s: B = %d < 0", fn, B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "%s: gamma = %d outside [1, %d]", fn, gamma, DSPARK_MAX_GAMMA);
  if (B > DSPARK_MAX_BATCH)
    return fail(DSPARK_E_UNSUPPORTED, "%s: B = %d exceeds %d", fn, B, DSPARK_MAX_BATCH);
  if (B > 0 && ((need_lens && !verify_lens) || !anchor_ids || !draft_tokens))
    return fail(DSPARK_E_INVALID, "%s: an input pointer is NULL", fn);
  if (!cu_seqlens || !packed_ids || !pack_meta)
    return fail(DSPARK_E_INVALID, "%s: an output pointer is NULL", fn);
  if (!tiers_host || num_tiers < 1 || num_tiers > DSPARK_MAX_TIERS)
    return fail(DSPARK_E_INVALID, "%s: need 1..%d tiers, got %d", fn, DSPARK_MAX_TIERS, num_tiers);
  if (tiers_host[0] < 1) return fail(DSPARK_E_INVALID, "%s: tiers must be >= 1", fn);
  for (int i = 1; i < num_tiers; ++i) {
    if (tiers_host[i] <= tiers_host[i - 1])
      return fail(DSPARK_E_INVALID, "%s: tiers not strictly ascending at %d", fn, i);
  }
  if ((int64_t)tiers_host[num_tiers - 1] < (int64_t)B * (gamma + 1))
    return fail(DSPARK_E_INVALID, "%s: last tier %d < B * (gamma + 1) = %lld", fn,
                tiers_host[num_tiers - 1], (long long)B * (gamma + 1));
  a->B = B;
  a->gamma = gamma;
  a->ntiers = num_tiers;
  a->lens = verify_lens;
  a->anchors = anchor_ids;
  a->drafts = draft_tokens;
  a->prefix = prefix_lens;
  a->cu = cu_seqlens;
  a->ids = packed_ids;
  a->req = packed_req;
  a->pos = packed_pos;
  a->meta = pack_meta;
  for (int i = 0; i < DSPARK_MAX_TIERS; ++i) a->tiers[i] = i < num_tiers ? tiers_host[i] : 0;
  return DSPARK_OK;
}

extern "C" {

dspark_status dspark_plan(int32_t B, int32_t gamma, dspark_input kind, const float* conf,
                          const float* sts_temp, int32_t min_verify_len,
                          int32_t max_verify_len, float survival_eps, int32_t budget_lo,
                          int32_t budget_hi, float cost_bias, const float* cost_alpha,
                          int32_t alpha_len, const float* cost_theta, int32_t theta_len,
                          int32_t* verify_lens, int32_t* plan_meta, double* plan_val,
                          float* survival_out, double* sweep_out, void* stream) {
  dspark::PlanArgs a;
  dspark_status st = check_plan("dspark_plan", B, gamma, kind, conf, sts_temp, min_verify_len,
                                max_verify_len, survival_eps, budget_lo, budget_hi, cost_bias,
                                cost_alpha, alpha_len, cost_theta, theta_len, verify_lens,
                                plan_meta, plan_val, survival_out, sweep_out, &a);
  if (st != DSPARK_OK) return st;
  return launched(dspark::launch_plan(a, nullptr, (hipStream_t)stream), "dspark_plan");
}

dspark_status dspark_plan_pack(int32_t B, int32_t gamma, dspark_input kind, const float* conf,
                               const float* sts_temp, int32_t min_verify_len,
                               int32_t max_verify_len, float survival_eps, int32_t budget_lo,
                               int32_t budget_hi, float cost_bias, const float* cost_alpha,
                               int32_t alpha_len, const float* cost_theta, int32_t theta_len,
                               int32_t* verify_lens, int32_t* plan_meta, double* plan_val,
                               float* survival_out, double* sweep_out, const int32_t* anchor_ids,
                               const int32_t* draft_tokens, const int32_t* tiers_host,
                               int32_t num_tiers, const int32_t* prefix_lens, int32_t* cu_seqlens,
                               int32_t* packed_ids, int32_t* packed_req, int32_t* packed_pos,
                               int32_t* pack_meta, void* stream) {
  dspark::PlanArgs a;
  dspark_status st = check_plan("dspark_plan_pack", B, gamma, kind, conf, sts_temp,
                                min_verify_len, max_verify_len, survival_eps, budget_lo,
                                budget_hi, cost_bias, cost_alpha, alpha_len, cost_theta,
                                theta_len, verify_lens, plan_meta, plan_val, survival_out,
                                sweep_out, &a);
  if (st != DSPARK_OK) return st;
  dspark::PackArgs p;
  st = check_pack("dspark_plan_pack", B, gamma, verify_lens, false, anchor_ids, draft_tokens,
                  tiers_host, num_tiers, prefix_lens, cu_seqlens, packed_ids, packed_req,
                  packed_pos, pack_meta, &p);
  if (st != DSPARK_OK) return st;
  return launched(dspark::launch_plan(a, &p, (hipStream_t)stream), "dspark_plan_pack");
}

dspark_status dspark_plan_pack_ex(int32_t B, int32_t gamma, dspark_input kind, const float* conf,
                                  const float* sts_temp, int32_t min_verify_len,
                                  int32_t max_verify_len, float survival_eps, int32_t budget_lo,
                                  int32_t budget_hi, float cost_bias, const float* cost_alpha,
                                  int32_t alpha_len, const float* cost_theta, int32_t theta_len,
                                  int32_t* verify_lens, int32_t* plan_meta, double* plan_val,
                                  float* survival_out, double* sweep_out,
                                  const int32_t* anchor_ids, const int32_t* draft_tokens,
                                  const int32_t* tiers_host, int32_t num_tiers,
                                  const int32_t* prefix_lens, int32_t* cu_seqlens,
                                  int32_t* packed_ids, int32_t* packed_req, int32_t* packed_pos,
                                  int32_t* pack_meta, const dspark_plan_options* options,
                                  void* stream) {
  dspark::PlanArgs a;
  dspark_status st = check_plan("dspark_plan_pack_ex", B, gamma, kind, conf, sts_temp,
                                min_verify_len, max_verify_len, survival_eps, budget_lo,
                                budget_hi, cost_bias, cost_alpha, alpha_len, cost_theta,
                                theta_len, verify_lens, plan_meta, plan_val, survival_out,
                                sweep_out, &a, options);
  if (st != DSPARK_OK) return st;
  dspark::PackArgs p;
  st = check_pack("dspark_plan_pack_ex", B, gamma, verify_lens, false, anchor_ids, draft_tokens,
                  tiers_host, num_tiers, prefix_lens, cu_seqlens, packed_ids, packed_req,
                  packed_pos, pack_meta, &p);
  if (st != DSPARK_OK) return st;
  return launched(dspark::launch_plan(a, &p, (hipStream_t)stream), "dspark_plan_pack_ex");
}

dspark_status dspark_pack(int32_t B, int32_t gamma, const int32_t* verify_lens,
                          const int32_t* anchor_ids, const int32_t* draft_tokens,
                          const int32_t* tiers_host, int32_t num_tiers,
                          const int32_t* prefix_lens, int32_t* cu_seqlens,
                          int32_t* packed_ids, int32_t* packed_req, int32_t* packed_pos,
                          int32_t* pack_meta, void* stream) {
  dspark::PackArgs a;
  dspark_status st = check_pack("dspark_pack", B, gamma, verify_lens, true, anchor_ids,
                                draft_tokens, tiers_host, num_tiers, prefix_lens, cu_seqlens,
                                packed_ids, packed_req, packed_pos, pack_meta, &a);
  if (st != DSPARK_OK) return st;
  return launched(dspark::launch_pack(a, (hipStream_t)stream), "dspark_pack");
}

dspark_status dspark_cap_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                const void* strided_logits, int64_t ld,
                                const int32_t* verify_lens, const int32_t* draft_tokens,
                                const int32_t* prefix_lens, int32_t* row_argmax, int32_t* ceiling,
                                int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                int32_t* out_tokens, int32_t* new_seq_lens, uint8_t* prefix_mask,
                                int32_t* accept_meta, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (B < 0) return fail(DSPARK_E_INVALID, "dspark_cap_accept: B = %d < 0", B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "dspark_cap_accept: gamma = %d outside [1, %d]", gamma,
                DSPARK_MAX_GAMMA);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16)
    return fail(DSPARK_E_UNSUPPORTED, "dspark_cap_accept: unsupported dtype %d", (int)dt);
  if (V < 1 || V > DSPARK_MAX_VOCAB)
    return fail(V < 1 ? DSPARK_E_INVALID : DSPARK_E_UNSUPPORTED,
                "dspark_cap_accept: V = %d outside [1, %d]", V, DSPARK_MAX_VOCAB);
  if (ld < V)
    return fail(DSPARK_E_INVALID, "dspark_cap_accept: ld = %lld < V = %d", (long long)ld, V);
  const size_t es = elem_size(dt);
  if ((ld * (int64_t)es) % 16 != 0)
    return fail(DSPARK_E_INVALID,
                "dspark_cap_accept: row stride %lld bytes is not a multiple of 16",
                (long long)(ld * (int64_t)es));
  const int64_t rows64 = (int64_t)B * (gamma + 1);
  const RowGeom g = row_geom(V, dt);
  if (rows64 * g.chunks > 0x7fffffffLL)
    return fail(DSPARK_E_UNSUPPORTED, "dspark_cap_accept: B * (gamma + 1) * chunks overflows int32");
  const int rows = (int)rows64;
  if (!accept_meta) return fail(DSPARK_E_INVALID, "dspark_cap_accept: accept_meta is NULL");
  if (B > 0) {
    if (!strided_logits || !aligned16(strided_logits))
      return fail(DSPARK_E_INVALID, "dspark_cap_accept: strided_logits NULL or not 16-byte aligned");
    if (!verify_lens || !draft_tokens || !row_argmax || !ceiling || !num_correct || !bonus ||
        !commit_lens || !out_tokens)
      return fail(DSPARK_E_INVALID, "dspark_cap_accept: a required pointer is NULL");
  }
  if (new_seq_lens && !prefix_lens)
    return fail(DSPARK_E_INVALID, "dspark_cap_accept: new_seq_lens needs prefix_lens");
  const size_t need = ws_bytes(rows, g.chunks);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return fail(DSPARK_E_WORKSPACE,
                "dspark_cap_accept: workspace needs %zu bytes, 256-byte aligned", need);

  dspark::AcceptArgs a;
  a.logits = static_cast<const unsigned char*>(strided_logits);
  a.ld_bytes = ld * (int64_t)es;
  a.V = V;
  a.max_rows = rows;
  a.B = B;
  a.gamma = gamma;
  a.fixed_rows = rows;
  a.chunks = g.chunks;
  a.chunk_vecs = g.chunk_vecs;
  a.nvec = g.nvec;
  a.tail = g.tail;
  a.cu = nullptr;
  a.drafts = draft_tokens;
  a.prefix = prefix_lens;
  a.row_am = row_argmax;
  a.num_correct = num_correct;
  a.bonus = bonus;
  a.commit = commit_lens;
  a.out_tokens = out_tokens;
  a.new_seq = new_seq_lens;
  a.mask = prefix_mask;
  a.meta = accept_meta;
  a.partials = static_cast<unsigned long long*>(workspace);
  a.lens = verify_lens;
  a.ceiling = ceiling;
  const int64_t units = (int64_t)rows * g.chunks;
  const int grid = units > 0 ? (int)units : 1;
  return launched(dspark::launch_accept(a, dt, grid, (hipStream_t)stream), "dspark_cap_accept");
}

dspark_status dspark_scatter_to_strided(int32_t B, int32_t stride, const int32_t* cu_seqlens,
                                        int32_t max_rows, const void* packed,
                                        int64_t packed_ld_bytes, void* strided,
                                        int64_t strided_ld_bytes, int64_t row_bytes,
                                        int32_t* scatter_meta, void* stream) {
  if (B < 0) return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: B = %d < 0", B);
  if (stride < 1 || stride > DSPARK_MAX_GAMMA + 1)
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: stride = %d outside [1, %d]", stride,
                DSPARK_MAX_GAMMA + 1);
  if (max_rows < 0)
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: max_rows = %d < 0", max_rows);
  if (row_bytes < 1 || row_bytes > (1LL << 30))
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: row_bytes = %lld outside [1, 2^30]",
                (long long)row_bytes);
  if (packed_ld_bytes < row_bytes || strided_ld_bytes < row_bytes ||
      packed_ld_bytes % 16 != 0 || strided_ld_bytes % 16 != 0)
    return fail(DSPARK_E_INVALID,
                "dspark_scatter_to_strided: row strides must be >= row_bytes and multiples of 16");
  if (!cu_seqlens || !scatter_meta)
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: cu_seqlens or scatter_meta is NULL");
  if (B > 0 && (!strided || !aligned16(strided)))
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: strided NULL or not 16-byte aligned");
  if (max_rows > 0 && (!packed || !aligned16(packed)))
    return fail(DSPARK_E_INVALID, "dspark_scatter_to_strided: packed NULL or not 16-byte aligned");
  dspark::ScatterArgs a;
  a.src = static_cast<const unsigned char*>(packed);
  a.src_ld = packed_ld_bytes;
  a.dst = static_cast<unsigned char*>(strided);
  a.dst_ld = strided_ld_bytes;
  a.B = B;
  a.stride = stride;
  a.max_rows = max_rows;
  a.nvec = (int)(row_bytes / 16);
  a.tail = (int)(row_bytes % 16);
  const int max_unit = dspark::kScatterThreads * dspark::kScatterVecsPerThread;
  a.chunks = std::max(1, (a.nvec + max_unit - 1) / max_unit);
  a.chunk_vecs = (a.nvec + a.chunks - 1) / a.chunks;
  a.cu = cu_seqlens;
  a.meta = scatter_meta;
  if ((int64_t)B * a.chunks > 0x7fffffffLL)
    return fail(DSPARK_E_UNSUPPORTED, "dspark_scatter_to_strided: B * units overflows int32");
  return launched(dspark::launch_scatter(a, (hipStream_t)stream), "dspark_scatter_to_strided");
}

size_t dspark_sts_workspace_size(int32_t N, int32_t gamma, int32_t n_t, int32_t n_bins) {
  if (N < 0 || N > DSPARK_STS_MAX_RECORDS || gamma < 1 || gamma > DSPARK_MAX_GAMMA || n_t < 1 ||
      n_t > DSPARK_STS_MAX_GRID || n_bins < 1 || n_bins > DSPARK_STS_MAX_BINS)
    return 0;
  return sts_geom(N, n_t, n_bins).bytes;
}

dspark_status dspark_sts_fit(int32_t N, int32_t gamma, const float* z, const uint8_t* prefix_mask,
                             const float* t_grid_host, int32_t n_t, int32_t n_bins, float* temps,
                             int32_t* t_index, double* ece, double* brier, double* ece_grid,
                             float* survival_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (N < 0 || N > DSPARK_STS_MAX_RECORDS)
    return fail(N < 0 ? DSPARK_E_INVALID : DSPARK_E_UNSUPPORTED,
                "dspark_sts_fit: N = %d outside [0, %d]", N, DSPARK_STS_MAX_RECORDS);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "dspark_sts_fit: gamma = %d outside [1, %d]", gamma,
                DSPARK_MAX_GAMMA);
  if (!t_grid_host || n_t < 1 || n_t > DSPARK_STS_MAX_GRID)
    return fail(DSPARK_E_INVALID, "dspark_sts_fit: need 1..%d grid temperatures, got %d",
                DSPARK_STS_MAX_GRID, n_t);
  for (int t = 0; t < n_t; ++t) {
    if (!(t_grid_host[t] > 0.0f && t_grid_host[t] <= FLT_MAX))
      return fail(DSPARK_E_INVALID, "dspark_sts_fit: grid temperature %d is not positive and finite",
                  t);
  }
  if (n_bins < 1 || n_bins > DSPARK_STS_MAX_BINS)
    return fail(DSPARK_E_INVALID, "dspark_sts_fit: n_bins = %d outside [1, %d]", n_bins,
                DSPARK_STS_MAX_BINS);
  if (N > 0 && (!z || !prefix_mask))
    return fail(DSPARK_E_INVALID, "dspark_sts_fit: z or prefix_mask is NULL");
  if (!temps || !t_index || !ece || !brier)
    return fail(DSPARK_E_INVALID, "dspark_sts_fit: an output pointer is NULL");
  const StsGeom g = sts_geom(N, n_t, n_bins);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < g.bytes)
    return fail(DSPARK_E_WORKSPACE, "dspark_sts_fit: workspace needs %zu bytes, 256-byte aligned",
                g.bytes);
  dspark::StsArgs a;
  a.N = N;
  a.gamma = gamma;
  a.n_t = n_t;
  a.nbins = n_bins;
  a.per_block = g.per_block;
  a.n_blocks = g.n_blocks;
  a.z = z;
  a.labels = prefix_mask;
  for (int t = 0; t < DSPARK_STS_MAX_GRID; ++t) a.grid[t] = t < n_t ? t_grid_host[t] : 0.0f;
  a.temps = temps;
  a.t_index = t_index;
  a.ece = ece;
  a.brier = brier;
  a.ece_grid = ece_grid;
  a.surv_out = survival_out;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.s_work[0] = reinterpret_cast<float*>(ws + g.s_off[0]);
  a.s_work[1] = reinterpret_cast<float*>(ws + g.s_off[1]);
  a.hists = reinterpret_cast<long long*>(ws + g.h_off);
  return launched(dspark::launch_sts(a, (hipStream_t)stream), "dspark_sts_fit");
}

size_t dspark_accept_workspace_size(int32_t max_rows, int32_t V, dspark_dtype dt) {
  if (max_rows < 0 || V < 1 || V > DSPARK_MAX_VOCAB) return 0;
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return 0;
  return ws_bytes(max_rows, row_geom(V, dt).chunks);
}

namespace {

// The body of dspark_accept, with the partials in `workspace` (null: the
// no-allocation variant, whose partials go to the library's own array).
dspark_status accept_call(const char* fn, int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                          const void* packed_logits, int64_t ld, int32_t max_rows,
                          const int32_t* cu_seqlens, const int32_t* draft_tokens,
                          const int32_t* prefix_lens, int32_t* row_argmax, int32_t* num_correct,
                          int32_t* bonus, int32_t* commit_lens, int32_t* out_tokens,
                          int32_t* new_seq_lens, uint8_t* prefix_mask, int32_t* accept_meta,
                          void* workspace, size_t workspace_bytes, bool own_scratch,
                          void* stream) {
  if (B < 0) return fail(DSPARK_E_INVALID, "%s: B = %d < 0", fn, B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "%s: gamma = %d outside [1, %d]", fn, gamma,
                DSPARK_MAX_GAMMA);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16)
    return fail(DSPARK_E_UNSUPPORTED, "%s: unsupported dtype %d", fn, (int)dt);
  if (V < 1 || V > DSPARK_MAX_VOCAB)
    return fail(V < 1 ? DSPARK_E_INVALID : DSPARK_E_UNSUPPORTED,
                "%s: V = %d outside [1, %d]", fn, V, DSPARK_MAX_VOCAB);
  if (max_rows < 0) return fail(DSPARK_E_INVALID, "%s: max_rows = %d < 0", fn, max_rows);
  if (ld < V) return fail(DSPARK_E_INVALID, "%s: ld = %lld < V = %d", fn, (long long)ld, V);
  const size_t es = elem_size(dt);
  if ((ld * (int64_t)es) % 16 != 0)
    return fail(DSPARK_E_INVALID, "%s: row stride %lld bytes is not a multiple of 16", fn,
                (long long)(ld * (int64_t)es));
  if (max_rows > 0 && (!packed_logits || !aligned16(packed_logits)))
    return fail(DSPARK_E_INVALID, "%s: packed_logits NULL or not 16-byte aligned", fn);
  if (!cu_seqlens || !accept_meta)
    return fail(DSPARK_E_INVALID, "%s: cu_seqlens or accept_meta is NULL", fn);
  if (B > 0 && (!draft_tokens || !num_correct || !bonus || !commit_lens || !out_tokens))
    return fail(DSPARK_E_INVALID, "%s: a required per-request pointer is NULL", fn);
  if (max_rows > 0 && !row_argmax)
    return fail(DSPARK_E_INVALID, "%s: row_argmax is NULL", fn);
  if (new_seq_lens && !prefix_lens)
    return fail(DSPARK_E_INVALID, "%s: new_seq_lens needs prefix_lens", fn);
  const RowGeom g = row_geom(V, dt);
  if ((int64_t)max_rows * g.chunks > 0x7fffffffLL)
    return fail(DSPARK_E_UNSUPPORTED, "%s: max_rows * chunks overflows int32", fn);
  const size_t need = ws_bytes(max_rows, g.chunks);
  if (own_scratch) {
    if (need > DSPARK_NOALLOC_SCRATCH_BYTES)
      return fail(DSPARK_E_WORKSPACE,
                  "%s: max_rows = %d at V = %d needs %zu bytes of partials, above the %d-byte "
                  "array of the no-allocation entry point; use dspark_accept with a workspace",
                  fn, max_rows, V, need, DSPARK_NOALLOC_SCRATCH_BYTES);
    const hipError_t e = noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return fail(DSPARK_E_LAUNCH, "%s: resolving the scratch array on this device: %s", fn,
                  hipGetErrorString(e));
  } else if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
             workspace_bytes < need) {
    return fail(DSPARK_E_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn, need);
  }

  dspark::AcceptArgs a;
  a.logits = static_cast<const unsigned char*>(packed_logits);
  a.ld_bytes = ld * (int64_t)es;
  a.V = V;
  a.max_rows = max_rows;
  a.B = B;
  a.gamma = gamma;
  a.chunks = g.chunks;
  a.chunk_vecs = g.chunk_vecs;
  a.nvec = g.nvec;
  a.tail = g.tail;
  a.cu = cu_seqlens;
  a.drafts = draft_tokens;
  a.prefix = prefix_lens;
  a.row_am = row_argmax;
  a.num_correct = num_correct;
  a.bonus = bonus;
  a.commit = commit_lens;
  a.out_tokens = out_tokens;
  a.new_seq = new_seq_lens;
  a.mask = prefix_mask;
  a.meta = accept_meta;
  a.partials = static_cast<unsigned long long*>(workspace);
  a.fixed_rows = -1;
  a.lens = nullptr;
  a.ceiling = nullptr;
  // one workgroup per (row, unit) of the largest possible packed total; the
  // kernel reads the actual total on the device and idle workgroups exit
  const int64_t units_max = (int64_t)max_rows * g.chunks;
  const int grid = units_max > 0 ? (int)units_max : 1;
  return launched(dspark::launch_accept(a, dt, grid, (hipStream_t)stream), fn);
}

}  // namespace

dspark_status dspark_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                            const void* packed_logits, int64_t ld, int32_t max_rows,
                            const int32_t* cu_seqlens, const int32_t* draft_tokens,
                            const int32_t* prefix_lens, int32_t* row_argmax,
                            int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                            int32_t* out_tokens, int32_t* new_seq_lens, uint8_t* prefix_mask,
                            int32_t* accept_meta, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return accept_call("dspark_accept", B, gamma, V, dt, packed_logits, ld, max_rows, cu_seqlens,
                     draft_tokens, prefix_lens, row_argmax, num_correct, bonus, commit_lens,
                     out_tokens, new_seq_lens, prefix_mask, accept_meta, workspace,
                     workspace_bytes, false, stream);
}

dspark_status dspark_accept_noalloc(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                    const void* packed_logits, int64_t ld, int32_t max_rows,
                                    const int32_t* cu_seqlens, const int32_t* draft_tokens,
                                    const int32_t* prefix_lens, int32_t* row_argmax,
                                    int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                    int32_t* out_tokens, int32_t* new_seq_lens,
                                    uint8_t* prefix_mask, int32_t* accept_meta, void* stream) {
  return accept_call("dspark_accept_noalloc", B, gamma, V, dt, packed_logits, ld, max_rows,
                     cu_seqlens, draft_tokens, prefix_lens, row_argmax, num_correct, bonus,
                     commit_lens, out_tokens, new_seq_lens, prefix_mask, accept_meta, nullptr, 0,
                     true, stream);
}

size_t dspark_accept_sampling_workspace_size(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt) {
  if (B < 0 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || V < 1 || V > DSPARK_MAX_VOCAB ||
      (dt != DSPARK_F32 && dt != DSPARK_BF16))
    return 0;
  const SampGeom g = samp_geom(B, gamma, V, dt);
  if ((int64_t)B * (2 * gamma + 1) * g.chunks > 0x7fffffffLL) return 0;
  return g.bytes;
}

dspark_status dspark_accept_sampling(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                     const void* packed_logits, int64_t ld, int32_t max_rows,
                                     const int32_t* cu_seqlens, const void* draft_logits,
                                     int64_t ld_q, const int32_t* draft_tokens,
                                     const float* temperatures, const uint32_t* rand_accept,
                                     const uint32_t* rand_sample, const int32_t* prefix_lens,
                                     int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                     int32_t* out_tokens, int32_t* new_seq_lens,
                                     int32_t* accept_meta, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const char* fn = "dspark_accept_sampling";
  if (B < 0) return fail(DSPARK_E_INVALID, "%s: B = %d < 0", fn, B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "%s: gamma = %d outside [1, %d]", fn, gamma, DSPARK_MAX_GAMMA);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16)
    return fail(DSPARK_E_UNSUPPORTED, "%s: unsupported dtype %d", fn, (int)dt);
  if (V < 1 || V > DSPARK_MAX_VOCAB)
    return fail(V < 1 ? DSPARK_E_INVALID : DSPARK_E_UNSUPPORTED, "%s: V = %d outside [1, %d]", fn,
                V, DSPARK_MAX_VOCAB);
  if (max_rows < 0) return fail(DSPARK_E_INVALID, "%s: max_rows = %d < 0", fn, max_rows);
  const SampGeom sg = samp_geom(B, gamma, V, dt);
  if ((int64_t)B * (2 * gamma + 1) * sg.chunks > 0x7fffffffLL ||
      (int64_t)max_rows + (int64_t)B * gamma > 0x7fffffffLL)
    return fail(DSPARK_E_UNSUPPORTED, "%s: B, gamma and V give too many work units", fn);
  if (ld < V || ld_q < V)
    return fail(DSPARK_E_INVALID, "%s: ld = %lld or ld_q = %lld below V = %d", fn, (long long)ld,
                (long long)ld_q, V);
  const size_t es = elem_size(dt);
  if ((ld * (int64_t)es) % 16 != 0 || (ld_q * (int64_t)es) % 16 != 0)
    return fail(DSPARK_E_INVALID, "%s: a row stride is not a multiple of 16 bytes", fn);
  if (max_rows > 0 && (!packed_logits || !aligned16(packed_logits)))
    return fail(DSPARK_E_INVALID, "%s: packed_logits NULL or not 16-byte aligned", fn);
  if (B > 0 && (!draft_logits || !aligned16(draft_logits)))
    return fail(DSPARK_E_INVALID, "%s: draft_logits NULL or not 16-byte aligned", fn);
  if (!cu_seqlens || !accept_meta)
    return fail(DSPARK_E_INVALID, "%s: cu_seqlens or accept_meta is NULL", fn);
  if (B > 0 && (!draft_tokens || !temperatures || !rand_accept || !rand_sample || !num_correct ||
                !bonus || !commit_lens || !out_tokens))
    return fail(DSPARK_E_INVALID, "%s: a required per-request pointer is NULL", fn);
  if (new_seq_lens && !prefix_lens)
    return fail(DSPARK_E_INVALID, "%s: new_seq_lens needs prefix_lens", fn);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < sg.bytes)
    return fail(DSPARK_E_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn,
                sg.bytes);
  const RowGeom g = row_geom(V, dt);
  dspark::SampArgs a;
  a.tgt = static_cast<const unsigned char*>(packed_logits);
  a.ld_t = ld * (int64_t)es;
  a.drf = static_cast<const unsigned char*>(draft_logits);
  a.ld_q = ld_q * (int64_t)es;
  a.V = V;
  a.nvec = g.nvec;
  a.tail = g.tail;
  a.chunks = sg.chunks;
  a.chunk_vecs = sg.chunk_vecs;
  a.max_rows = max_rows;
  a.B = B;
  a.gamma = gamma;
  a.cu = cu_seqlens;
  a.drafts = draft_tokens;
  a.temps = temperatures;
  a.ra = rand_accept;
  a.rs = rand_sample;
  a.prefix = prefix_lens;
  a.num_correct = num_correct;
  a.bonus = bonus;
  a.commit = commit_lens;
  a.out_tokens = out_tokens;
  a.new_seq = new_seq_lens;
  a.meta = accept_meta;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.kpart = reinterpret_cast<unsigned long long*>(ws);
  a.zpart = reinterpret_cast<unsigned long long*>(ws + sg.part_bytes);
  a.rpart = reinterpret_cast<unsigned long long*>(ws + 2 * sg.part_bytes);
  a.jobs = reinterpret_cast<dspark::SampJob*>(ws + 2 * sg.part_bytes + sg.rpart_bytes);
  return launched(dspark::launch_sampling(a, dt, (hipStream_t)stream), fn);
}

dspark_status dspark_tv_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                               const void* draft_logits, int64_t ld_q,
                               const void* target_logits, int64_t ld_p,
                               int32_t target_rows_per_req, float* accept_rate,
                               float* survival, void* stream) {
  if (B < 0) return fail(DSPARK_E_INVALID, "dspark_tv_accept: B = %d < 0", B);
  if (gamma < 1 || gamma > DSPARK_MAX_GAMMA)
    return fail(DSPARK_E_INVALID, "dspark_tv_accept: gamma = %d outside [1, %d]", gamma,
                DSPARK_MAX_GAMMA);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16)
    return fail(DSPARK_E_UNSUPPORTED, "dspark_tv_accept: unsupported dtype %d", (int)dt);
  if (V < 1 || V > DSPARK_MAX_VOCAB)
    return fail(V < 1 ? DSPARK_E_INVALID : DSPARK_E_UNSUPPORTED,
                "dspark_tv_accept: V = %d outside [1, %d]", V, DSPARK_MAX_VOCAB);
  if ((int64_t)B * gamma > 0x7fffffffLL)
    return fail(DSPARK_E_UNSUPPORTED, "dspark_tv_accept: B * gamma too large");
  if (target_rows_per_req < gamma)
    return fail(DSPARK_E_INVALID, "dspark_tv_accept: target_rows_per_req %d < gamma %d",
                target_rows_per_req, gamma);
  if (ld_q < V || ld_p < V)
    return fail(DSPARK_E_INVALID, "dspark_tv_accept: row stride below V");
  const size_t es = elem_size(dt);
  if ((ld_q * (int64_t)es) % 16 != 0 || (ld_p * (int64_t)es) % 16 != 0)
    return fail(DSPARK_E_INVALID, "dspark_tv_accept: row strides must be multiples of 16 bytes");
  if (B > 0) {
    if (!draft_logits || !target_logits || !aligned16(draft_logits) || !aligned16(target_logits))
      return fail(DSPARK_E_INVALID, "dspark_tv_accept: logits NULL or not 16-byte aligned");
    if (!accept_rate || !survival)
      return fail(DSPARK_E_INVALID, "dspark_tv_accept: an output pointer is NULL");
  }
  const int epv = (int)(16 / es);
  dspark::TvArgs a;
  a.q = static_cast<const unsigned char*>(draft_logits);
  a.ldq_bytes = ld_q * (int64_t)es;
  a.p = static_cast<const unsigned char*>(target_logits);
  a.ldp_bytes = ld_p * (int64_t)es;
  a.V = V;
  a.B = B;
  a.gamma = gamma;
  a.rows_per_req = target_rows_per_req;
  a.nvec = V / epv;
  a.tail = V - a.nvec * epv;
  a.a_out = accept_rate;
  a.s_out = survival;
  return launched(dspark::launch_tv(a, dt, (hipStream_t)stream), "dspark_tv_accept");
}

}  // extern "C"
