/*
 * dspark.h - C ABI of the DSpark per-step verify path for AMD Instinct MI355X
 * (gfx950).
 *
 * One decode step of confidence-scheduled speculative decoding, for B
 * requests that each drafted gamma tokens:
 *
 *   dspark_plan      STS confidence -> prefix survival -> global top-b budget
 *                    sweep -> verify_lens
 *   dspark_pack      verify_lens -> cu_seqlens, front-packed verify rows,
 *                    packed total rounded up to a captured tier
 *   dspark_plan_pack both of the above in one launch
 *   dspark_plan_pack_ex  the same with the 1D SPS cost model and/or graph-tier
 *                    alignment of the executed budget
 *   dspark_accept    packed target logits -> per-row argmax -> leading-match
 *                    count, bonus token, commit lengths, output tokens
 *   dspark_cap_accept    greedy accept on the full strided block, committing
 *                    at most verify_len - 1 drafts and reporting the uncapped
 *                    ceiling (cap-accept mode)
 *   dspark_scatter_to_strided  packed verify rows (logits or hidden states)
 *                    back to the strided [B, stride] layout
 *   dspark_sts_fit   (offline) the per-position STS temperatures that feed
 *                    dspark_plan, fitted on recorded logits and prefix_masks
 *   dspark_accept_sampling  chain speculative-sampling accept (temperature > 0;
 *                    temperature 0 requests take the greedy rule)
 *   dspark_tv_accept (optional) soft accept-rate 1 - TV(softmax q, softmax p)
 *                    and its per-request cumulative product, which can feed
 *                    dspark_plan as survivals
 *
 * Page references used below:
 *   [Budget] akiyangdev, "DSpark 自适应 Verify 怎样分配候选预算"
 *   [Round]  akiyangdev, "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit"
 *   [SGLang] yingzheng, "DSpark 接入 SGLang：用置信度驱动可变长度验证"
 *   [CSSD]   charlestar, "DSpark confidence-scheduled speculative decoding"
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers to caller-owned memory, except those
 *     whose name ends in _host. The library never allocates, frees or
 *     synchronizes. Each call enqueues its kernels on `stream` (a hipStream_t
 *     passed as void*; NULL is the null stream) and returns at once, so a
 *     step can be captured into a HIP graph.
 *   - Integers are int32 and arrays are dense, request-major and row-major:
 *     conf[r * gamma + (k - 1)] holds draft position k = 1..gamma of
 *     request r. Verify row j = 0 of a request is its root (anchor) row;
 *     row j >= 1 verifies draft j.
 *   - Argument errors are found on the host before any launch and returned
 *     synchronously; nothing is enqueued then. Data errors only visible on
 *     the device (bad cost table, NaN confidence, malformed lengths) are
 *     reported in the status word of the *_meta output, together with a
 *     documented fallback. Kernels never trap.
 *   - dspark_last_error() returns a thread-local description of the last
 *     non-OK status returned on the calling thread.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dspark_status {
  DSPARK_OK = 0,
  DSPARK_E_INVALID = 1,     /* bad scalar argument or missing required pointer */
  DSPARK_E_UNSUPPORTED = 2, /* sizes beyond what the kernels handle (see limits) */
  DSPARK_E_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  DSPARK_E_LAUNCH = 4       /* the HIP runtime refused a launch */
} dspark_status;

typedef enum dspark_dtype { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* What dspark_plan's `conf` holds. */
typedef enum dspark_input {
  DSPARK_IN_CONF_LOGITS = 0, /* confidence logits z; c = sigmoid(z / T[k]) */
  DSPARK_IN_COND = 1,        /* conditional confidences c in [0, 1] */
  DSPARK_IN_SURVIVAL = 2     /* prefix survivals s in [0, 1], non-increasing in k */
} dspark_input;

/* Bits of the device-side status word (plan_meta[2], pack_meta[2],
 * accept_meta[1]). */
#define DSPARK_DATA_BAD_COST 1 /* some T(B, M) (or SPS) <= 0 or non-finite in the
                                  sweep, or SPS probes not strictly ascending */
#define DSPARK_DATA_BAD_CONF 2 /* confidence/survival/temperature out of domain */
#define DSPARK_DATA_BAD_LENS 4 /* verify lengths or cu_seqlens malformed */
#define DSPARK_DATA_BAD_LOGITS 8 /* a row a sampling request reads holds NaN or
                                    +inf, or has no finite maximum */

/* Limits. */
#define DSPARK_MAX_GAMMA 64
#define DSPARK_MAX_CANDIDATES 8192 /* B * gamma for dspark_plan */
#define DSPARK_MAX_BATCH 8192      /* B for dspark_plan and dspark_pack */
#define DSPARK_MAX_TIERS 32
#define DSPARK_MAX_VOCAB 262144
#define DSPARK_MAX_SPS_PROBES 512
#define DSPARK_STS_MAX_GRID 128        /* temperature candidates of dspark_sts_fit */
#define DSPARK_STS_MAX_BINS 64         /* calibration bins of dspark_sts_fit */
#define DSPARK_STS_MAX_RECORDS 4194304 /* records of dspark_sts_fit */

/* How the planner prices a budget (see dspark_plan_pack_ex). */
typedef enum dspark_cost_mode {
  DSPARK_COST_ADDITIVE = 0, /* objective tau(b) / T, T = bias + alpha[B] + theta[M] */
  DSPARK_COST_SPS1D = 1     /* objective tau(b) * SPS(M), SPS by floor lookup */
} dspark_cost_mode;

/* Options of dspark_plan_pack_ex (host memory; the arrays are device memory). */
typedef struct dspark_plan_options {
  dspark_cost_mode cost_mode;
  const int32_t* sps_m;  /* SPS1D: [sps_len] probe totals M, strictly ascending */
  const float* sps;      /* SPS1D: [sps_len] steps per second at each probe */
  int32_t sps_len;       /* SPS1D: 1..DSPARK_MAX_SPS_PROBES */
  int32_t align_to_tier; /* nonzero: graph-tier alignment (paid-padding reclamation) */
} dspark_plan_options;

/*
 * dspark_plan - choose the extra verify budget and the per-request verify_lens.
 *
 * Defined by [Budget] §一 (tau(b) = B + sum of the b largest survivals;
 * budget = argmax_b tau(b) / T(B, B + b); ties in survival go to the earlier
 * position, then the lower request id; ScheduleVerifyLensTopk allocation
 * with min/max_verify_len and survival_eps), [Budget] §二 (STS runtime
 * c_k = sigmoid(z_k / T_k), S_k = prod_{i<=k} c_i), [Budget] §四 and [CSSD]
 * (additive cost T(B, M) = bias + alpha(B) + theta(M), M = bs + K).
 *
 * Arithmetic (the same on every GPU and in the CPU reference):
 *   x = RN32(z / T[k]); c = the float32 nearest to 1 / (1 + e^-x);
 *   s_1 = c_1, s_k = RN32(s_{k-1} * c_k).
 *   L_min = clamp(min_verify_len, 1, gamma + 1);
 *   L_max = clamp(max_verify_len, L_min, gamma + 1).
 *   Positions k < L_min are always verified and their survivals count in tau.
 *   Candidates are positions L_min <= k < L_max with s >= survival_eps,
 *   sorted by (s descending, k ascending, r ascending).
 *   tau(b) = B + sum over forced + the first b candidates, each term taken
 *   at a resolution of 2^-40 (nearest, ties to even): exact and
 *   order-independent.
 *   T(b) = (bias + alpha[B]) + theta[B * L_min + b], summed in fp64;
 *   ratio(b) = tau(b) / T(b) in fp64.
 *   b* = the smallest b in [budget_lo, budget_hi] (clipped to
 *   [0, #candidates]) with the largest ratio.
 *   verify_lens[r] = L_min + #{candidates of r among the first b*}.
 *
 * Arguments:
 *   B                  requests, 0 <= B <= DSPARK_MAX_BATCH,
 *                      B * gamma <= DSPARK_MAX_CANDIDATES
 *   gamma              drafted positions per request, 1..DSPARK_MAX_GAMMA
 *   kind, conf         [B, gamma] float32 as given by `kind`
 *   sts_temp           [gamma] float32 STS temperatures (CONF_LOGITS only;
 *                      otherwise ignored, may be NULL)
 *   min_verify_len, max_verify_len   clamped as above
 *   survival_eps       candidates below it are dropped (equal is kept)
 *   budget_lo, budget_hi  extra-row budget range; budget_hi < 0 means no
 *                      upper limit; budget_lo > budget_hi >= 0 is invalid
 *   cost_bias          ms
 *   cost_alpha         [alpha_len] float32, alpha(bs) in ms; alpha_len > B
 *   cost_theta         [theta_len] float32, theta(M) in ms for M = 0..;
 *                      theta_len > B * L_max
 *   verify_lens        out [B] int32
 *   plan_meta          out [4] int32: b*, #candidates, status bits,
 *                      B * L_min + b* (total verify rows before tier rounding)
 *   plan_val           out [2] double: tau(b*), ratio(b*) (tokens per ms)
 *   survival_out       out [B, gamma] float32 survivals, or NULL
 *   sweep_out          out [B * gamma + 1][2] double (tau(b), ratio(b)) for
 *                      b = 0..#candidates and NaN beyond, or NULL
 * Data errors: a bad cost value at a considered budget sets
 *   DSPARK_DATA_BAD_COST. A NaN/out-of-range confidence or survival, an
 *   increasing survival, or a non-positive/non-finite temperature sets
 *   DSPARK_DATA_BAD_CONF. Either way verify_lens = L_max for every request
 *   (the static window), plan_meta = {-1, -1, status, B * L_max},
 *   plan_val = NaN and sweep_out = NaN.
 */
dspark_status dspark_plan(int32_t B, int32_t gamma, dspark_input kind, const float* conf,
                          const float* sts_temp, int32_t min_verify_len,
                          int32_t max_verify_len, float survival_eps, int32_t budget_lo,
                          int32_t budget_hi, float cost_bias, const float* cost_alpha,
                          int32_t alpha_len, const float* cost_theta, int32_t theta_len,
                          int32_t* verify_lens, int32_t* plan_meta, double* plan_val,
                          float* survival_out, double* sweep_out, void* stream);

/*
 * dspark_pack - compact ragged verify layout.
 *
 * Defined by [Budget] §五 and §六 (compact RaggedVerifyLayout; cu_seqlens_q
 * is the exclusive prefix sum of verify_lens with a leading 0, e.g.
 * [2,1,4] -> [0,2,3,7]), [Round] §三 (verify ids are the anchor followed by
 * the drafts; compact mode front-packs the anchor plus the selected draft
 * prefix), [SGLang] and [CSSD] (the packed total is rounded up to the
 * smallest captured tier that holds it).
 *
 *   cu_seqlens[0] = 0, cu_seqlens[r+1] = cu_seqlens[r] + verify_lens[r]
 *   row cu[r] + j (j < verify_lens[r]): packed_ids = j ? draft_tokens[r, j-1]
 *     : anchor_ids[r]; packed_req = r; packed_pos = prefix_lens[r] + j
 *     (just j if prefix_lens is NULL)
 *   pad rows [total, tier): packed_ids = 0, packed_req = -1, packed_pos = 0
 *
 * Arguments:
 *   B, gamma           as for dspark_plan (B <= DSPARK_MAX_BATCH)
 *   verify_lens        [B] int32, each in [1, gamma + 1]
 *   anchor_ids         [B] int32 root-row token per request
 *   draft_tokens       [B, gamma] int32
 *   tiers_host         HOST array of num_tiers int32, strictly ascending,
 *                      1 <= num_tiers <= DSPARK_MAX_TIERS, first >= 1,
 *                      last >= B * (gamma + 1); read during the call only
 *   prefix_lens        [B] int32 or NULL
 *   cu_seqlens         out [B + 1] int32
 *   packed_ids         out, capacity tiers_host[num_tiers - 1] int32
 *   packed_req, packed_pos  out, same capacity, or NULL
 *   pack_meta          out [3] int32: total, tier, status bits
 * Only rows [0, tier) are written.
 * Data errors: a length outside [1, gamma + 1] sets DSPARK_DATA_BAD_LENS and
 * is clamped into that range before packing.
 */
dspark_status dspark_pack(int32_t B, int32_t gamma, const int32_t* verify_lens,
                          const int32_t* anchor_ids, const int32_t* draft_tokens,
                          const int32_t* tiers_host, int32_t num_tiers,
                          const int32_t* prefix_lens, int32_t* cu_seqlens,
                          int32_t* packed_ids, int32_t* packed_req, int32_t* packed_pos,
                          int32_t* pack_meta, void* stream);

/*
 * dspark_plan_pack - dspark_plan followed by dspark_pack in one launch.
 *
 * Same arithmetic, arguments and outputs as dspark_plan, then dspark_pack
 * on the verify_lens just computed (their ragged layout, tier and packed
 * rows), in the same workgroup. This saves one kernel launch per step.
 * verify_lens is written as by dspark_plan and packed from the same values.
 * In the bad-data fallback the static window L_max is packed.
 * Argument rules are the union of both calls. Pack's own status bit is
 * never set here, because planned lengths are always in range.
 */
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
                               int32_t* pack_meta, void* stream);

/*
 * dspark_plan_pack_ex - dspark_plan_pack with a choice of cost model and
 * optional graph-tier alignment.
 *
 * Defined by [Budget] §一 (the objective tau(b) * SPS(B + b) with a
 * one-dimensional SPS table, or tau(b) / T(B, B + b) with the additive one;
 * budget = argmax_b), [Budget] §四 (the 1D SpsCostTable: steps per second
 * measured at probe totals M and read by floor lookup, the nearest probe at
 * or below M with no interpolation, so a cliff in the table is kept), and
 * [Budget] §五 and §三 (graph-tier alignment: the executed budget is filled
 * up to the graph tier the chosen budget already pays for, with the next
 * candidates by survival; it never enters the next tier and never adds rows
 * that are not candidates).
 *
 * options == NULL gives dspark_plan_pack exactly. Otherwise:
 *   cost_mode DSPARK_COST_SPS1D: objective(b) = RN64(tau(b) * SPS(M)),
 *     M = B * L_min + b; a total below the first probe takes the first
 *     probe's value. cost_bias, cost_alpha and cost_theta are ignored (the
 *     table pointers may be NULL). Probes that are not strictly ascending, or
 *     an SPS that is not positive and finite at a considered b, set
 *     DSPARK_DATA_BAD_COST (fallback as in dspark_plan).
 *   align_to_tier: with b* the argmax and t the smallest tier >= B * L_min +
 *     b*, the executed budget is b_exec = min(b* + t - (B * L_min + b*),
 *     number of candidates); verify_lens and the packed rows follow the top
 *     b_exec candidates. budget_hi bounds b* only.
 * Outputs as dspark_plan_pack; plan_meta[0] is b*, plan_meta[3] the executed
 * total B * L_min + b_exec, plan_val and sweep_out hold tau and the
 * objective.
 */
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
                                  void* stream);

/*
 * dspark_accept - greedy accept over packed target logits.
 *
 * Defined by [Round] §四 and §五 (AcceptGreedy: target_predict =
 * argmax(target_logits); draft k is checked against the prediction of verify
 * row k-1; correct_len counts the leading matches and stops at the first
 * mismatch; bonus is the prediction of the last valid input row;
 * FinalizeAcceptLens commit_lens = correct_len + 1 and new_seq_lens =
 * prefix_lens + commit_lens; BuildOutTokens out[:, :gamma] = drafts, then
 * out[r, correct_len] = bonus), [Budget] §二 (prefix_mask = positions <
 * num_correct_drafts) and [Budget] §三 (the cap: at most verify_len - 1
 * drafts can be accepted).
 *
 * The argmax compares values as float32 (bfloat16 widens exactly). -0 equals
 * +0, NaN ranks above every number, and the lowest index wins ties.
 * out_tokens[r, gamma] starts at -1.
 *
 * Arguments:
 *   B, gamma, V        requests, drafted positions, vocabulary
 *                      (1 <= V <= DSPARK_MAX_VOCAB)
 *   dt                 element type of packed_logits
 *   packed_logits      [max_rows, ld] rows; 16-byte aligned; ld * element
 *                      size a multiple of 16 bytes; ld >= V
 *   max_rows           rows the logits buffer holds (>= the packed total;
 *                      rows at or beyond it are never read)
 *   cu_seqlens         [B + 1] int32 as written by dspark_pack; the total
 *                      cu_seqlens[B] is read on the device
 *   draft_tokens       [B, gamma] int32
 *   prefix_lens        [B] int32 or NULL (then new_seq_lens must be NULL)
 *   row_argmax         out [max_rows] int32; rows < total are written
 *   num_correct, bonus, commit_lens   out [B] int32
 *   out_tokens         out [B, gamma + 1] int32
 *   new_seq_lens       out [B] int32 or NULL
 *   prefix_mask        out [B, gamma] uint8 or NULL
 *   accept_meta        out [2] int32: cu_seqlens[B], status bits
 *   workspace          device scratch of dspark_accept_workspace_size() bytes,
 *                      256-byte aligned; its contents on entry do not matter
 *                      and it carries no state between calls. Calls that
 *                      share a workspace must not overlap in time.
 * Data errors: a request whose rows are not 1..gamma+1 rows inside
 *   [0, min(cu_seqlens[B], max_rows)) sets DSPARK_DATA_BAD_LENS and gets
 *   num_correct 0, bonus -1, commit 0, out_tokens -1, prefix_mask 0,
 *   new_seq = prefix.
 */
dspark_status dspark_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                            const void* packed_logits, int64_t ld, int32_t max_rows,
                            const int32_t* cu_seqlens, const int32_t* draft_tokens,
                            const int32_t* prefix_lens, int32_t* row_argmax,
                            int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                            int32_t* out_tokens, int32_t* new_seq_lens, uint8_t* prefix_mask,
                            int32_t* accept_meta, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * dspark_accept_noalloc - dspark_accept without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, outputs, data errors and stream behaviour are those of
 * dspark_accept, without workspace and workspace_bytes. The per-unit partials
 * live in a device array of DSPARK_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; the call allocates and frees
 * nothing. It accepts max_rows while dspark_accept_workspace_size(max_rows, V,
 * dt) <= DSPARK_NOALLOC_SCRATCH_BYTES (max_rows <= 16384 at V = 129280 bf16,
 * 4096 at V = 262144 f32); beyond that it returns DSPARK_E_WORKSPACE without
 * launching anything. The first call on a device looks up the array's address
 * on that device (the device current at the call); a failure there returns
 * DSPARK_E_LAUNCH.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * partials: calls that overlap in time on one GPU (on different streams, or
 * from different host threads without ordering) race on it and give undefined
 * results. Calls ordered on one stream are safe. Nothing needs clearing: each
 * call rewrites every partial it reads.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES (1 << 20)
dspark_status dspark_accept_noalloc(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                    const void* packed_logits, int64_t ld, int32_t max_rows,
                                    const int32_t* cu_seqlens, const int32_t* draft_tokens,
                                    const int32_t* prefix_lens, int32_t* row_argmax,
                                    int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                    int32_t* out_tokens, int32_t* new_seq_lens,
                                    uint8_t* prefix_mask, int32_t* accept_meta, void* stream);

/*
 * dspark_cap_accept - greedy accept in cap-accept mode.
 *
 * Defined by [SGLang] "三种 verify mode" and "可观测性" (cap-accept verifies
 * the full drafted block but commits only inside the scheduler's window, so
 * its output equals compact mode's while it also exposes how many tokens full
 * verification would have accepted), [CSSD] "static、compact 与 cap-accept
 * 三种模式", and [Budget] §五 (the target keeps the fixed B * (gamma + 1)
 * rows; correct_len is clipped to verify_len - 1 at accept time).
 *
 * Rows are strided: request r's verify row j (j = 0..gamma, row 0 the root)
 * is row r * (gamma + 1) + j. The argmax and the leading-match rule are those
 * of dspark_accept; the count runs over all gamma drafts (the ceiling), then
 *   num_correct = min(ceiling, verify_len - 1), bonus = prediction of row
 *   num_correct, and the remaining outputs as in dspark_accept.
 *
 * Arguments (as dspark_accept unless stated):
 *   strided_logits     [B * (gamma + 1), ld] rows, 16-byte aligned
 *   verify_lens        [B] int32 (the planner's lengths)
 *   row_argmax         out [B * (gamma + 1)] int32, every row written
 *   ceiling            out [B] int32, uncapped leading matches (0..gamma)
 *   accept_meta        out [2] int32: B * (gamma + 1), status bits
 *   workspace          dspark_accept_workspace_size(B * (gamma + 1), V, dt)
 *                      bytes, 256-byte aligned, contents irrelevant
 * Data errors: a verify length outside [1, gamma + 1] sets
 *   DSPARK_DATA_BAD_LENS and gives that request the outputs of a malformed
 *   request of dspark_accept; its ceiling is still written.
 */
dspark_status dspark_cap_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                const void* strided_logits, int64_t ld,
                                const int32_t* verify_lens, const int32_t* draft_tokens,
                                const int32_t* prefix_lens, int32_t* row_argmax, int32_t* ceiling,
                                int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                int32_t* out_tokens, int32_t* new_seq_lens, uint8_t* prefix_mask,
                                int32_t* accept_meta, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * dspark_scatter_to_strided - copy front-packed rows back to stride.
 *
 * Defined by [Round] §三 (ScatterCompactToStrided: after the target forward,
 * logits and hidden states of the compact rows are restored to the uniform
 * [bs x stride] logical layout so that accept can address fixed positions;
 * rows that were not verified are not recomputed and verify_lens still says
 * which results are valid).
 *
 *   strided[r * stride + j] = packed[cu_seqlens[r] + j]
 *   for j < cu_seqlens[r + 1] - cu_seqlens[r]; other strided rows are not
 *   written.
 *
 * Arguments:
 *   B, stride          requests; strided rows per request (1..gamma_max + 1)
 *   cu_seqlens         [B + 1] int32, as written by dspark_pack
 *   max_rows           rows the packed buffer holds; rows at or beyond it are
 *                      never read
 *   packed             packed rows, packed_ld_bytes apart; 16-byte aligned
 *   strided            destination rows, strided_ld_bytes apart; 16-byte
 *                      aligned; must not overlap `packed`
 *   row_bytes          bytes copied per row (any element type or width: e.g.
 *                      V * element size for logits, H * element size for
 *                      hidden states); both strides >= row_bytes and
 *                      multiples of 16
 *   scatter_meta       out [2] int32: cu_seqlens[B], status bits
 * Data errors: a request whose rows are not 1..stride rows inside
 *   [0, min(cu_seqlens[B], max_rows)) sets DSPARK_DATA_BAD_LENS and none of
 *   its rows is written.
 */
dspark_status dspark_scatter_to_strided(int32_t B, int32_t stride, const int32_t* cu_seqlens,
                                        int32_t max_rows, const void* packed,
                                        int64_t packed_ld_bytes, void* strided,
                                        int64_t strided_ld_bytes, int64_t row_bytes,
                                        int32_t* scatter_meta, void* stream);

/* Bytes of workspace dspark_accept needs for `max_rows` rows of V elements of
 * type dt (0 for invalid sizes). */
size_t dspark_accept_workspace_size(int32_t max_rows, int32_t V, dspark_dtype dt);

/*
 * dspark_accept_sampling - chain speculative-sampling accept over packed
 * target logits.
 *
 * Defined by [Round] §五 (AcceptSampling: acceptance by speculative sampling
 * over the draft-side probabilities that actually proposed each draft and
 * the target probabilities, giving correct_len and the bonus), [Budget] §二
 * (a draft drawn from q is accepted with probability min(1, p/q); the mean
 * acceptance is sum_x min(p, q) = 1 - TV) and [CSSD] "截短为什么不会改变目标分布"
 * (accept, reject and the residual resample follow the speculative
 * algorithm; random numbers keep their meaning under compaction).
 *
 * Request r owns packed rows cu[r] .. cu[r+1]-1 (l rows). With T =
 * temperatures[r]:
 *   T == 0   greedy: exactly dspark_accept's rule (argmax ties, NaN order).
 *   T > 0    drafts k = 1..l-1 in order: p is target row k-1, q is draft row
 *            r * gamma + k - 1 (the distribution that proposed draft k),
 *            both at temperature T. The first rejected draft k ends the
 *            chain with num_correct = k - 1 and the token of column k - 1
 *            drawn from the residual max(0, p - q) of that pair; if all pass,
 *            column l - 1 gets a token drawn from p of target row l - 1.
 * Probabilities as integer weights, so every decision is an exact integer
 * comparison: for a row x with maximum m, t = RN32((x - m) * c + 31) in one
 * fused multiply-add with c = RN32(K / T) * 2^-16 and K = 94548.4609375 (the
 * float32 nearest to 2^16 log2 e), and W = 2^t from the hardware base-2
 * exponential, rounded to the nearest integer. p = W / sum W, each weight
 * within 4e-6 relative plus half a unit of 2^31 exp((x - m) / T).
 *   accept draft d  iff  (rand_accept >> 8) * Wq[d] * Zp < 2^24 * Wp[d] * Zq
 *   draw from integer weights w (total S) with word v: the smallest index
 *   whose running sum exceeds floor((v >> 8) * S / 2^24); residual weights
 *   max(0, Wp * Zq - Wq * Zp), and if they are all 0, w = Wp.
 * A draft outside [0, V) is rejected.
 *
 * Arguments:
 *   B, gamma, V, dt    as for dspark_accept
 *   packed_logits      [max_rows, ld] target rows, as for dspark_accept
 *   max_rows           rows the target buffer holds
 *   cu_seqlens         [B + 1] int32; the total cu_seqlens[B] is read on the
 *                      device
 *   draft_logits       [B * gamma, ld_q] draft rows (row r * gamma + k - 1
 *                      proposed draft k), same dtype; 16-byte aligned, ld_q *
 *                      element size a multiple of 16, ld_q >= V
 *   draft_tokens       [B, gamma] int32
 *   temperatures       [B] float32: 0 for greedy, > 0 for sampling
 *   rand_accept        [B, gamma] uint32 random words; [r, k-1] tests draft k
 *   rand_sample        [B, gamma + 1] uint32; [r, c] draws the token of
 *                      output column c. A word w stands for the uniform
 *                      (w >> 8) / 2^24.
 *   prefix_lens        [B] int32 or NULL (then new_seq_lens must be NULL)
 *   num_correct, bonus, commit_lens   out [B] int32
 *   out_tokens         out [B, gamma + 1] int32 (drafts, the drawn token at
 *                      column num_correct, -1 after)
 *   new_seq_lens       out [B] int32 or NULL
 *   accept_meta        out [2] int32: cu_seqlens[B], status bits
 *   workspace          dspark_accept_sampling_workspace_size(B, gamma, V, dt) bytes,
 *                      256-byte aligned; no state between calls; calls that
 *                      share it must not overlap in time.
 * Data errors: a malformed layout (as for dspark_accept) sets
 *   DSPARK_DATA_BAD_LENS; a negative, NaN or infinite temperature sets
 *   DSPARK_DATA_BAD_CONF; a row the sampling request reads with a NaN or
 *   +inf, or with every element -inf, sets DSPARK_DATA_BAD_LOGITS. Such a
 *   request gets num_correct 0, bonus -1, commit 0, out_tokens -1 and
 *   new_seq = prefix.
 */
dspark_status dspark_accept_sampling(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                                     const void* packed_logits, int64_t ld, int32_t max_rows,
                                     const int32_t* cu_seqlens, const void* draft_logits,
                                     int64_t ld_q, const int32_t* draft_tokens,
                                     const float* temperatures, const uint32_t* rand_accept,
                                     const uint32_t* rand_sample, const int32_t* prefix_lens,
                                     int32_t* num_correct, int32_t* bonus, int32_t* commit_lens,
                                     int32_t* out_tokens, int32_t* new_seq_lens,
                                     int32_t* accept_meta, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Bytes of workspace dspark_accept_sampling needs (0 for invalid sizes). */
size_t dspark_accept_sampling_workspace_size(int32_t B, int32_t gamma, int32_t V,
                                             dspark_dtype dt);

/*
 * dspark_tv_accept - soft accept-rate and its cumulative product.
 *
 * Defined by [Budget] §二 (DeepSpec target: accept_rate = 1 - 0.5 *
 * sum |softmax(draft_logits) - softmax(target_logits)|, equal to
 * sum_x min(p, q) under rejection sampling; confidence_prefix_targets =
 * accept_rate.cumprod).
 *
 *   a[r, k] = sum_x min(softmax(q_{r,k})_x, softmax(p_{r,k-1})_x), clamped to
 *   [0, 1]; S[r, k] = RN32(S[r, k-1] * a[r, k]).
 * The draft row that proposed draft k pairs with target row k-1, the row that
 * predicts position k.
 *
 * Arguments:
 *   B, gamma, V, dt    as for dspark_accept
 *   draft_logits       q rows: row r * gamma + (k - 1); stride ld_q elements
 *   target_logits      p rows: row r * target_rows_per_req + (k - 1); stride ld_p
 *   target_rows_per_req >= gamma (gamma + 1 for the strided verify layout)
 *   Both logit buffers: 16-byte aligned, ld * element size multiple of 16.
 *   accept_rate        out [B, gamma] float32
 *   survival           out [B, gamma] float32 (usable as DSPARK_IN_SURVIVAL)
 * Accuracy: float32 with exp2/log2 hardware approximations; within 1e-5
 * absolute of an fp64 evaluation for the vocabularies above.
 */
dspark_status dspark_tv_accept(int32_t B, int32_t gamma, int32_t V, dspark_dtype dt,
                               const void* draft_logits, int64_t ld_q,
                               const void* target_logits, int64_t ld_p,
                               int32_t target_rows_per_req, float* accept_rate,
                               float* survival, void* stream);

/*
 * dspark_sts_fit - fit the per-position STS temperatures on recorded data.
 *
 * Defined by [Budget] §二 (runtime STS c_k = sigmoid(z_k / T_k), S_k =
 * prod_{i<=k} c_i; the fitter searches a positive temperature per position,
 * in order, keeping the cumulative survival already fitted for the earlier
 * positions, and keeps the candidate with the lower expected calibration
 * error against the greedy prefix label) and [CSSD] "为什么置信度必须校准"
 * (ECE = sum_b |I_b| / n * |acc(I_b) - conf(I_b)| over confidence bins; a
 * position's label is only meaningful given that the earlier ones survived).
 *
 * For k = 1..gamma in order and every candidate T of t_grid_host:
 *   S_k(T) = RN32(S_{k-1} * sigmoid32(RN32(z[n, k-1] / T))), S_0 = 1,
 *   n * ECE_k(T) = sum_b |#labels in b - sum of S_k(T) in b| with bins
 *   b = min(floor(S * n_bins), n_bins - 1) and each S taken at 2^-40
 *   resolution (nearest), so the comparison is exact;
 * T_k = the candidate with the smallest ECE (the first one on ties), and
 * S_k = S_k(T_k). sigmoid32 is the correctly rounded sigmoid of dspark_plan.
 * The labels are the prefix_mask that dspark_accept writes: prefix_mask[n,
 * k-1] nonzero means draft k of record n was accepted.
 *
 * Arguments:
 *   N, gamma           records (0..DSPARK_STS_MAX_RECORDS), positions (1..64)
 *   z                  [N, gamma] float32 confidence logits
 *   prefix_mask        [N, gamma] uint8 labels
 *   t_grid_host        HOST [n_t] float32 candidates, each > 0 and finite
 *                      (1 <= n_t <= DSPARK_STS_MAX_GRID)
 *   n_bins             1..DSPARK_STS_MAX_BINS
 *   temps              out [gamma] float32 chosen temperatures
 *   t_index            out [gamma] int32 their grid indices
 *   ece, brier         out [gamma] float64: ECE and Brier score (mean of
 *                      (S - label)^2, each term at 2^-40) of the chosen S_k
 *   ece_grid           out [gamma, n_t] float64 ECE of every candidate, or NULL
 *   survival_out       out [N, gamma] float32 fitted S_k, or NULL
 *   workspace          dspark_sts_workspace_size() bytes, 256-byte aligned;
 *                      contents irrelevant, no state between calls; calls
 *                      that share it must not overlap in time
 * Errors: argument errors only. Infinite logits give survivals 0 or 1; a NaN
 *   logit gives a NaN survival, which is binned and summed as 0.
 */
dspark_status dspark_sts_fit(int32_t N, int32_t gamma, const float* z, const uint8_t* prefix_mask,
                             const float* t_grid_host, int32_t n_t, int32_t n_bins, float* temps,
                             int32_t* t_index, double* ece, double* brier, double* ece_grid,
                             float* survival_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Bytes of workspace dspark_sts_fit needs (0 for invalid sizes). */
size_t dspark_sts_workspace_size(int32_t N, int32_t gamma, int32_t n_t, int32_t n_bins);

/* Name of a status code (static string). */
const char* dspark_status_str(dspark_status s);

/* Thread-local detail of the last non-OK status on this thread ("" if none). */
const char* dspark_last_error(void);

/* ABI version: (major << 16) | minor. */
int32_t dspark_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
