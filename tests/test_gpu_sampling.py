"""GPU parity of dspark_accept_sampling against the CPU oracle, through the C ABI.

The bars:

* the definition (``oracle.sampling``, float64 softmaxes, accept iff
  U < p(d) / q(d), the normalised residual max(0, p - q)), on every case:
  every GPU decision equals the float64 one unless the random number lies
  inside the error band the kernels' weights allow (``prob_error_bound``),
  where either decision is valid and the check follows the GPU's; greedy,
  malformed and out-of-domain requests match exactly, and so does the status
  word. Band cases are counted and reported;
* the kernels' weights themselves against 2^31 exp((x - m) / T) in float64:
  single weights isolated in crafted rows, and every slot's weight sum, each
  within the per-weight bound (EPS_W relative plus half a unit) the band is
  built on.
"""

import json
import math
import os
from pathlib import Path

import numpy as np
import pytest
import torch

import dspark_verify_scheduling_amd as dv
import oracle
from oracle import sampling as F64
from oracle.accept import as_f32_rows
from workloads import gen
from _gpu import DEV, logits_up, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _bits(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint32)).view(np.int32)


def run_gpu(B, gamma, V, dt, tgt, drf, cu, drafts, temps, ra, rs, prefix=None, max_rows=None,
            tag=""):
    """tgt [>= cu[B], V] and drf [B * gamma, V] as float32 or bf16 bits."""
    max_rows = tgt.shape[0] if max_rows is None else max_rows
    say(f"accept_sampling {tag} B={B} gamma={gamma} V={V} dt={dt} rows={max_rows}")
    ld = V if (V * (2 if dt == dv.BF16 else 4)) % 16 == 0 else None
    if ld is None:  # pad rows to a 16-byte stride
        per = 8 if dt == dv.BF16 else 4
        ld = (V + per - 1) // per * per
        pad = lambda x: np.pad(x, ((0, 0), (0, ld - V)))
        tgt, drf = pad(tgt), pad(drf)
    out = dv.alloc_sampling_outputs(B, gamma, V, dt, DEV)
    for t in (out.num_correct, out.bonus, out.commit_lens, out.out_tokens, out.new_seq_lens):
        t.fill_(-9)
    dv.dspark_accept_sampling(
        B, gamma, V, dt, logits_up(tgt, dt), ld, max_rows, up(np.asarray(cu, np.int32)),
        logits_up(drf if B else np.zeros((1, ld), tgt.dtype), dt), ld,
        up(np.asarray(drafts, np.int32).reshape(B, gamma)), up(np.asarray(temps, np.float32)),
        up(_bits(ra).reshape(B, gamma)), up(_bits(rs).reshape(B, gamma + 1)),
        up(np.asarray(prefix if prefix is not None else np.zeros(B), np.int32)), out)
    torch.cuda.synchronize()
    return {"num_correct": out.num_correct.cpu().numpy(), "bonus": out.bonus.cpu().numpy(),
            "commit": out.commit_lens.cpu().numpy(), "new_seq": out.new_seq_lens.cpu().numpy(),
            "out_tokens": out.out_tokens.cpu().numpy(), "meta": out.accept_meta.cpu().numpy()}


def check_status(got, ref, total):
    """accept_meta = [total, status], the status as the float64 oracle's."""
    assert got["meta"][0] == total and got["meta"][1] == ref["status"], (got["meta"], ref["status"])


def rand_case(seed, B, gamma, V, dt, greedy_frac=0.2, q_noise=0.5):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, gamma + 2, B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    tgt = rng.normal(0, 2.5, (total + 2, V)).astype(np.float32)
    drf = np.empty((B * gamma, V), np.float32)
    drafts = np.empty((B, gamma), np.int32)
    for r in range(B):
        for k in range(gamma):
            src = tgt[cu[r] + k] if k < lens[r] else rng.normal(0, 2.5, V)
            drf[r * gamma + k] = src + rng.normal(0, q_noise, V)
            # the draft is drawn from its own q (temperature 1)
            q = np.exp(drf[r * gamma + k] - drf[r * gamma + k].max())
            drafts[r, k] = rng.choice(V, p=q / q.sum())
    temps = rng.uniform(0.5, 1.5, B).astype(np.float32)
    temps[rng.random(B) < greedy_frac] = 0.0
    ra = rng.integers(0, 2**32, (B, gamma), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, gamma + 1), dtype=np.uint64).astype(np.uint32)
    prefix = rng.integers(5, 500, B).astype(np.int32)
    if dt == dv.BF16:
        tgt, drf = gen.f32_to_bf16_bits(tgt), gen.f32_to_bf16_bits(drf)
    return dict(B=B, gamma=gamma, V=V, dt=dt, tgt=tgt, drf=drf, cu=cu, drafts=drafts,
                temps=temps, ra=ra, rs=rs, prefix=prefix)


def check_f64(got, B, gamma, tgt, drf, dtype, cu, drafts, temps, ra, rs, prefix=None,
              max_rows=None, reqs=None, tag=""):
    """The GPU outputs against the float64 definition, band cases allowed."""
    rep = F64.validate(B, gamma, tgt, drf, dtype, cu, drafts, temps, ra, rs, got,
                       prefix_lens=prefix, max_rows=max_rows, reqs=reqs)
    st = rep["stats"]
    say(f"float64 {tag}: {st['sampling_requests']} sampling requests, "
        f"{st['accept_tests']} accept tests ({st['accept_band']} in the band, "
        f"{st['accept_band_flips']} decided otherwise), "
        f"{st['draws_p'] + st['draws_residual']} draws "
        f"({st['draws_p_band'] + st['draws_residual_band']} in the band, "
        f"{st['draws_p_flips'] + st['draws_residual_flips']} drew another token)")
    assert rep["failures"] == [], rep["failures"][:5]
    return st


def both(c, tag, max_rows=None):
    got = run_gpu(c["B"], c["gamma"], c["V"], c["dt"], c["tgt"], c["drf"], c["cu"], c["drafts"],
                  c["temps"], c["ra"], c["rs"], c["prefix"], max_rows=max_rows, tag=tag)
    dtype = "bf16" if c["dt"] == dv.BF16 else "f32"
    ref = F64.accept_sampling(c["B"], c["gamma"], c["tgt"], c["drf"], dtype, c["cu"],
                              c["drafts"], c["temps"], c["ra"], c["rs"], prefix_lens=c["prefix"],
                              max_rows=max_rows)
    check_status(got, ref, int(c["cu"][-1]))
    check_f64(got, c["B"], c["gamma"], c["tgt"], c["drf"], dtype, c["cu"], c["drafts"],
              c["temps"], c["ra"], c["rs"], c["prefix"], max_rows=max_rows, tag=tag)
    return got, ref


@pytest.mark.parametrize("seed,B,gamma,V,dt", [
    (1, 12, 4, 1000, dv.F32),
    (2, 16, 6, 4096, dv.BF16),
    (3, 9, 8, 4099, dv.BF16),   # ragged tail of 3 elements
    (4, 7, 3, 777, dv.F32),     # ragged tail of 1
    (5, 20, 5, 20000, dv.BF16), # several register slots
    (6, 5, 64, 300, dv.F32),    # gamma = 64: 65 rows and columns
])
def test_sampling_parity_small(seed, B, gamma, V, dt):
    c = rand_case(seed, B, gamma, V, dt)
    got, ref = both(c, f"seed={seed}")
    say(f"correct {got['num_correct'].tolist()[:12]} temps {np.round(c['temps'][:12], 2).tolist()}")


def test_sampling_parity_long_rows():
    # rows beyond the register-resident part: bf16 V > 131072, f32 V > 65536
    both(rand_case(7, 3, 3, 200003, dv.BF16, greedy_frac=0.0), "bf16 long rows")
    both(rand_case(8, 3, 3, 70001, dv.F32, greedy_frac=0.0), "f32 long rows")
    # the largest vocabulary the library takes
    both(rand_case(9, 2, 2, 262144, dv.BF16, greedy_frac=0.0), "bf16 rows of the maximum V")
    both(rand_case(10, 2, 2, 262144, dv.F32, greedy_frac=0.5), "f32 rows of the maximum V")


def test_all_greedy_equals_dspark_accept():
    w = gen.make(1)
    rng = np.random.default_rng(3)
    lens = rng.integers(1, w.gamma + 2, w.B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tgt = np.concatenate([w.target[r, :lens[r]] for r in range(w.B)])
    ex = gen.sampling_extras(w)
    drf = ex.draft_logits.reshape(w.B * w.gamma, w.V)
    got = run_gpu(w.B, w.gamma, w.V, dv.F32, tgt, drf, cu, w.drafts, np.zeros(w.B), ex.rand_accept,
                  ex.rand_sample, w.prefix_lens, tag="all greedy")
    ref = oracle.accept(w.B, w.gamma, tgt, "f32", cu, w.drafts, prefix_lens=w.prefix_lens)
    for k in ("num_correct", "bonus", "commit", "new_seq", "out_tokens"):
        assert np.array_equal(got[k], ref[k]), k


def test_sampling_edge_cases():
    c = rand_case(11, 8, 4, 512, dv.F32, greedy_frac=0.25)
    t = c["tgt"]
    t[c["cu"][1] + 1, 7] = np.nan         # request 1: NaN in a sampled row
    t[c["cu"][2], 3] = np.inf             # request 2: +inf
    t[c["cu"][3] + 0, :] = -np.inf        # request 3: no finite maximum
    c["temps"][[1, 2, 3]] = 1.0
    c["temps"][4] = -0.5                  # bad temperature
    c["temps"][5] = np.inf
    c["drafts"][6, 0] = c["V"] + 3        # outside the vocabulary
    c["drafts"][7, 1] = -1
    got, ref = both(c, "bad data")
    assert ref["status"] == F64.DATA_BAD_LOGITS | oracle.DATA_BAD_CONF
    # identical p and q rows: every draft in the support passes
    c = rand_case(12, 6, 5, 640, dv.BF16, greedy_frac=0.0)
    for r in range(c["B"]):
        for k in range(c["gamma"]):
            if c["cu"][r] + k < c["cu"][r + 1]:
                c["drf"][r * c["gamma"] + k] = c["tgt"][c["cu"][r] + k]
    got, _ = both(c, "p == q")
    assert np.array_equal(got["num_correct"], np.diff(c["cu"]) - 1)
    # malformed layout, and a total beyond max_rows
    c = rand_case(13, 6, 3, 256, dv.F32)
    c["cu"][3] = c["cu"][2]
    both(c, "empty request")
    c = rand_case(14, 6, 3, 256, dv.F32)
    both(c, "max_rows below the total", max_rows=int(c["cu"][-1]) - 2)
    # overlapping packed ranges (cu not increasing): requests 0 and 2 are each
    # well formed but share rows 3 and 4 at different temperatures; request 1
    # is malformed. Each valid request is decided at its own temperature.
    c = rand_case(16, 3, 5, 333, dv.BF16, greedy_frac=0.0)
    c["cu"] = np.array([0, 5, 3, 8], np.int32)
    if c["tgt"].shape[0] < 8:
        c["tgt"] = np.concatenate([c["tgt"]] * 4)[:10]
    c["temps"] = np.array([0.6, 1.0, 1.7], np.float32)
    got, ref = both(c, "overlapping ranges")
    assert ref["status"] == oracle.DATA_BAD_LENS and got["bonus"][0] >= 0 and got["bonus"][2] >= 0
    # a draw whose crossing point lies among the tail elements: all the mass
    # of the last target row on its final element (V = 4099 bf16: 3 tail elements)
    c = rand_case(17, 4, 3, 4099, dv.BF16, greedy_frac=0.0)
    for r in range(4):
        last = c["cu"][r + 1] - 1
        row = np.full(4099, -60.0, np.float32)
        row[4098] = 5.0
        c["tgt"][last] = gen.f32_to_bf16_bits(row)
    got, _ = both(c, "tail draw")
    # no requests
    c = rand_case(15, 1, 3, 256, dv.F32)
    got = run_gpu(0, 3, 256, dv.F32, c["tgt"][:4], np.zeros((0, 256), np.float32),
                  np.zeros(1, np.int32), np.zeros((0, 3)), np.zeros(0), np.zeros((0, 3)),
                  np.zeros((0, 4)), np.zeros(0), tag="B = 0")
    assert got["meta"].tolist() == [0, 0]


# Rows of 1024 to 16384 16-byte vectors take the one-read row-statistics
# kernel (persistent workgroups, rows held in 2, 4, 8 or 16 register slots per
# thread; more sampling rows than workgroups): its slot-count boundaries,
# ragged tails, greedy rows mixed in (which keep the per-unit maximum kernel),
# and rows whose maximum is not positive (exact keys) or is not finite.
@pytest.mark.parametrize("seed,B,gamma,V,dt,greedy", [
    (31, 40, 6, 10007, dv.BF16, 0.0),   # 1250 vectors: 2 slots, tail of 7, ~280 rows
    (32, 12, 4, 50000, dv.BF16, 0.3),   # 6250 vectors: 8 slots, greedy mixed in
    (33, 6, 3, 131072, dv.BF16, 0.0),   # 16384 vectors: 16 full slots
    (34, 9, 5, 8192, dv.BF16, 0.2),     # 1024 vectors: the smallest row it takes
    (35, 10, 4, 32001, dv.F32, 0.0),    # 8000 vectors and a tail of 1, float32
    (37, 16, 4, 32001, dv.F32, 0.5),    # float32 greedy rows: key, then index, merged
])
def test_sampling_rowstat_path(seed, B, gamma, V, dt, greedy):
    c = rand_case(seed, B, gamma, V, dt, greedy_frac=greedy)
    both(c, f"rowstat V={V}")


def test_sampling_rowstat_special_rows():
    c = rand_case(36, 10, 4, 10007, dv.BF16, greedy_frac=0.0)
    cu, V = c["cu"], c["V"]
    t32 = lambda row: gen.f32_to_bf16_bits(np.asarray(row, np.float32))
    rng = np.random.default_rng(36)
    c["tgt"][cu[0]] = t32(rng.normal(-20.0, 1.0, V))          # maximum below 0: exact keys
    row = np.full(V, -3.0, np.float32)
    row[V - 1] = 0.0                                            # maximum +0, in the tail
    c["tgt"][cu[1]] = t32(row)
    row = rng.normal(0, 2.0, V).astype(np.float32)
    row[V - 3] = 40.0                                           # maximum in the tail
    c["tgt"][cu[2]] = t32(row)
    c["drf"][3 * c["gamma"]] = t32(np.full(V, -1.5, np.float32))  # flat negative draft row
    c["tgt"][cu[4], 5] = 0x7FC0                                  # NaN
    c["tgt"][cu[5] + (1 if cu[6] - cu[5] > 1 else 0), V - 2] = 0x7F80  # +inf in the tail
    c["tgt"][cu[6]] = 0xFF80                                     # -inf row
    c["tgt"][cu[7], 100] = 0xFFC1                                # negative NaN
    got, ref = both(c, "rowstat special rows")
    assert ref["status"] & F64.DATA_BAD_LOGITS


def test_sampling_rowstat_greedy_special_rows():
    """Greedy rows in the row-statistics kernel: the first index of the
    maximum when the maximum is negative (exact keys, then the index from the
    same workgroup), tied, NaN (highest, first one wins) or in the tail."""
    c = rand_case(38, 8, 4, 10007, dv.BF16, greedy_frac=1.0)
    cu, V = c["cu"], c["V"]
    t32 = lambda row: gen.f32_to_bf16_bits(np.asarray(row, np.float32))
    rng = np.random.default_rng(38)
    c["tgt"][cu[0]] = t32(rng.normal(-20.0, 1.0, V))          # negative maximum
    row = np.full(V, -7.0, np.float32)
    row[[500, 9000, 9100]] = -2.0                               # negative, tied three times
    c["tgt"][cu[1]] = t32(row)
    row = rng.normal(0, 2.0, V).astype(np.float32)
    row[[77, 4000]] = 30.0                                      # positive tie
    c["tgt"][cu[2]] = t32(row)
    c["tgt"][cu[3], [900, 20]] = 0x7FC0                         # two NaNs: the first, 20
    row = rng.normal(0, 2.0, V).astype(np.float32)
    row[V - 2] = 50.0                                           # maximum in the tail
    c["tgt"][cu[4]] = t32(row)
    c["tgt"][cu[5], 33] = 0xFFC1                                # a negative NaN
    both(c, "rowstat greedy special rows")


def test_sampling_many_slots_two_read_path():
    """More than 64 slots per CU (B = 1000, gamma = 8: 17,000 slots) with rows
    the row-statistics kernel could hold (V = 8192 bf16): the batch keeps the
    two-read kernels. Every request is checked against the float64 definition."""
    B, G, V = 1000, 8, 8192
    rng = np.random.default_rng(41)
    lens = rng.integers(1, G + 2, B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    tgt = gen.f32_to_bf16_bits(rng.normal(0, 2.5, (total, V)).astype(np.float32))
    drf = gen.f32_to_bf16_bits(rng.normal(0, 2.5, (B * G, V)).astype(np.float32))
    drafts = rng.integers(0, V, (B, G)).astype(np.int32)
    temps = rng.uniform(0.5, 1.5, B).astype(np.float32)
    temps[rng.random(B) < 0.2] = 0.0
    ra = rng.integers(0, 2**32, (B, G), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, G + 1), dtype=np.uint64).astype(np.uint32)
    prefix = rng.integers(5, 500, B).astype(np.int32)
    got = run_gpu(B, G, V, dv.BF16, tgt, drf, cu, drafts, temps, ra, rs, prefix, tag="17000 slots")
    assert got["meta"].tolist() == [total, 0]
    check_f64(got, B, G, tgt, drf, "bf16", cu, drafts, temps, ra, rs, prefix,
              tag="17000 slots, all 1000 requests")


# the error summary is written only when DSPARK_SUMMARY_DIR names an existing folder
SUMMARY = Path(os.environ.get("DSPARK_SUMMARY_DIR", "/nonexistent")) / "sampling_f64_validation.json"


def _record(name, rec):
    """Add one workload's counts to the run's summary file (when the output
    folder exists: on a GPU run)."""
    if not SUMMARY.parent.is_dir():
        return
    data = json.loads(SUMMARY.read_text()) if SUMMARY.exists() else {}
    data[name] = rec
    SUMMARY.write_text(json.dumps(data, indent=1, sort_keys=True))


@pytest.mark.parametrize("cfg,greedy_frac", [(3, 0.0), (2, 0.1), (1, 0.1), (4, 0.1)])
def test_sampling_full_size_every_request(cfg, greedy_frac):
    """Full-size workloads (cfg1: B = 8, V = 32000 f32; cfg2: B = 64, V =
    151936 bf16; cfg3: B = 256, gamma = 8, V = 129280 bf16, the benchmark's
    own sampling inputs; cfg4: gamma = 16 with its own draft logits and a
    spread of verify lengths). cfg1-3 run on their planned layouts in the
    launch configuration the benchmark times (max_rows = the tier). Every
    request is checked against the float64 definition."""
    w = gen.make(cfg)
    if cfg == 4:
        lens = np.random.default_rng(4).integers(1, w.gamma + 2, w.B)
    else:
        p = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                        w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
        lens = p["verify_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    tgt = np.concatenate([w.target[r, :lens[r]] for r in range(w.B)])
    ex = gen.sampling_extras(w, greedy_frac=greedy_frac)
    drf = ex.draft_logits.reshape(w.B * w.gamma, w.V)
    max_rows = total if cfg == 4 else int(w.tiers[np.searchsorted(w.tiers, total)])
    tgt_pad = np.zeros((max_rows, w.V), tgt.dtype)
    tgt_pad[:total] = tgt
    dt = dv.BF16 if w.dtype == "bf16" else dv.F32
    got = run_gpu(w.B, w.gamma, w.V, dt, tgt_pad, drf, cu, w.drafts, ex.temps, ex.rand_accept,
                  ex.rand_sample, w.prefix_lens, tag=f"cfg{cfg} full")
    assert got["meta"].tolist() == [total, 0]
    st = check_f64(got, w.B, w.gamma, tgt_pad, drf, w.dtype, cu, w.drafts, ex.temps,
                   ex.rand_accept, ex.rand_sample, w.prefix_lens, max_rows=max_rows,
                   tag=f"cfg{cfg} all {w.B} requests")
    assert st["requests"] == w.B and st["sampling_requests"] == int(np.sum(ex.temps != 0))
    say(f"cfg{cfg}: mean correct {got['num_correct'].mean():.3f} over {w.B} requests, "
        f"{total} rows")
    if cfg == 3:  # a second call on the same inputs is identical (no state in the workspace)
        again = run_gpu(w.B, w.gamma, w.V, dt, tgt_pad, drf, cu, w.drafts, ex.temps,
                        ex.rand_accept, ex.rand_sample, w.prefix_lens, tag="cfg3 repeat")
        for k in ("num_correct", "bonus", "out_tokens"):
            assert np.array_equal(got[k], again[k])
    _record(f"cfg{cfg}", {"B": w.B, "gamma": w.gamma, "V": w.V, "dtype": w.dtype,
                          "rows": total, "max_rows": max_rows, "greedy_frac": greedy_frac, **st})


def test_sampling_graph_replay_matches_eager():
    """dspark_accept_sampling captured in a HIP graph: every replay, with new
    random words copied into the captured input buffers and eager calls in
    between, matches the eager result for those words."""
    c = rand_case(21, 24, 5, 3000, dv.BF16, greedy_frac=0.2)
    B, G, V = c["B"], c["gamma"], c["V"]
    tgt_t, drf_t = logits_up(c["tgt"], dv.BF16), logits_up(c["drf"], dv.BF16)
    cu_t, dr_t = up(c["cu"]), up(c["drafts"])
    tp_t, pf_t = up(c["temps"]), up(c["prefix"])
    ra_t, rs_t = up(_bits(c["ra"])), up(_bits(c["rs"]))
    out = dv.alloc_sampling_outputs(B, G, V, dv.BF16, DEV)
    rows = c["tgt"].shape[0]

    def call():
        dv.dspark_accept_sampling(B, G, V, dv.BF16, tgt_t, V, rows, cu_t, drf_t, V, dr_t, tp_t,
                                  ra_t, rs_t, pf_t, out)

    def snap():
        return [t.clone() for t in (out.num_correct, out.bonus, out.commit_lens, out.out_tokens,
                                    out.new_seq_lens, out.accept_meta)]

    rng = np.random.default_rng(5)
    words = [(rng.integers(0, 2**32, (B, G), dtype=np.uint64).astype(np.uint32),
              rng.integers(0, 2**32, (B, G + 1), dtype=np.uint64).astype(np.uint32))
             for _ in range(4)]
    expect = []
    for wa, ws in words:
        ra_t.copy_(up(_bits(wa)))
        rs_t.copy_(up(_bits(ws)))
        call()
        torch.cuda.synchronize()
        expect.append(snap())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("sampling graph: capture")
    with torch.cuda.graph(g):
        call()
    for i in range(8):
        wa, ws = words[i % 4]
        ra_t.copy_(up(_bits(wa)))
        rs_t.copy_(up(_bits(ws)))
        for t in (out.num_correct, out.bonus, out.out_tokens):
            t.fill_(-5)
        say(f"sampling graph: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snap(), expect[i % 4]):
            assert torch.equal(a, b), f"replay {i} differs"
        call()  # eager work between replays
        torch.cuda.synchronize()
    # and the words mattered: the four expected results are not all equal
    assert any(not torch.equal(expect[0][1], e[1]) for e in expect[1:])


# The weights themselves. The kernels leave per-chunk weight sums in the
# workspace; the layout read here is the library's internal one: per (slot,
# chunk) 64-bit maxima, then 64-bit weight sums, slots = B (gamma + 1) target
# slots then B gamma draft slots, chunks of 2048 16-byte vectors, each part
# padded to 256 bytes.
def _slot_sums(out, B, gamma, V, dt):
    esize = 2 if dt == dv.BF16 else 4
    chunks = max(1, -(-(V * esize // 16) // 2048))
    slots = B * (2 * gamma + 1)
    part_bytes = -(-(slots * chunks * 8) // 256) * 256
    ws = out.workspace.cpu().numpy()
    z = ws[part_bytes:part_bytes + slots * chunks * 8].view(np.uint64).reshape(slots, chunks)
    return [int(v) for v in z.astype(object).sum(axis=1)]


def _exact_weights(x, T):
    """2^31 exp((x - m) / T) in float64, m the row maximum (float32 values)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    return 2.0**31 * np.exp((x - np.max(x)) / np.float64(np.float32(T)))


@pytest.mark.parametrize("V,dt", [(1024, dv.F32), (4096, dv.F32)])
def test_sampling_single_weights_within_bound(V, dt):
    """Rows with the maximum at 0, one other finite element x and -inf
    elsewhere: a slot's weight sum is W(0) + W(x), so each call isolates one
    weight per slot. Over x from the maximum down past the last nonzero
    weight and temperatures from 0.05 to 4: W(max) = 2^31 exactly, and every
    W(x) within EPS_W relative plus half a unit of 2^31 exp(x / T). (V = 1024
    f32 takes the two-read kernels, V = 4096 the row-statistics kernel.)"""
    B, G = 32, 4
    rng = np.random.default_rng(V)
    lens = np.full(B, G + 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = B * (2 * G + 1)
    worst, n = 0.0, 0
    for it in range(6):
        temps = np.exp(rng.uniform(np.log(0.05), np.log(4.0), B)).astype(np.float32)
        # t* = 31 + x log2(e) / T spread over [-2, 31]
        frac = rng.uniform(-2.0, 31.0, slots)
        tgt = np.full((B * (G + 1), V), -np.inf, np.float32)
        drf = np.full((B * G, V), -np.inf, np.float32)
        xs = np.empty(slots, np.float32)
        for r in range(B):
            T = float(temps[r])
            for j in range(G + 1):
                sl = r * (G + 1) + j
                xs[sl] = np.float32((frac[sl] - 31.0) * T / math.log2(math.e))
                tgt[cu[r] + j, 0], tgt[cu[r] + j, 1 + sl % (V - 1)] = 0.0, min(xs[sl], 0.0)
            for k in range(G):
                sl = B * (G + 1) + r * G + k
                xs[sl] = np.float32((frac[sl] - 31.0) * T / math.log2(math.e))
                drf[r * G + k, 0], drf[r * G + k, 1 + sl % (V - 1)] = 0.0, min(xs[sl], 0.0)
        if it == 0:  # rows holding only the maximum
            tgt[cu[0], 1:] = -np.inf
            xs[0] = -np.inf
        drafts = np.zeros((B, G), np.int32)
        out = dv.alloc_sampling_outputs(B, G, V, dt, DEV)
        say(f"single weights V={V} call {it}")
        dv.dspark_accept_sampling(
            B, G, V, dt, logits_up(tgt, dt), V, tgt.shape[0], up(cu), logits_up(drf, dt), V,
            up(drafts), up(temps), up(np.zeros((B, G), np.int32)),
            up(np.zeros((B, G + 1), np.int32)), up(np.zeros(B, np.int32)), out)
        torch.cuda.synchronize()
        z = _slot_sums(out, B, G, V, dt)
        for sl in range(slots):
            r = sl // (G + 1) if sl < B * (G + 1) else (sl - B * (G + 1)) // G
            T = np.float64(temps[r])
            w = z[sl] - 2**31
            assert w >= 0, (sl, z[sl])
            x = np.float64(min(xs[sl], np.float32(0.0)))
            ws = 2.0**31 * math.exp(x / T) if np.isfinite(x) else 0.0
            bound = F64.EPS_W * ws + 0.5 + 1e-5
            assert abs(w - ws) <= bound, (sl, float(x), float(T), w, ws)
            if ws > 1e3:
                worst = max(worst, abs(w - ws) / ws)
            n += 1
    say(f"{n} single weights within the bound; largest relative error {worst:.3g} "
        f"(EPS_W = {F64.EPS_W:g})")


@pytest.mark.parametrize("seed,B,gamma,V,dt,t_lo,t_hi", [
    (21, 6, 4, 129280, dv.BF16, 0.3, 2.0),
    (22, 5, 3, 32000, dv.F32, 0.05, 1.5),   # small T: most weights near 0
    (23, 4, 5, 4099, dv.BF16, 0.5, 4.0),
])
def test_sampling_weight_sums_within_bound(seed, B, gamma, V, dt, t_lo, t_hi):
    """Every slot's weight sum Z against the float64 sum of 2^31 exp((x - m) /
    T): within the sum of the per-weight bounds."""
    c = rand_case(seed, B, gamma, V, dt, greedy_frac=0.0)
    rng = np.random.default_rng(seed + 100)
    c["temps"] = rng.uniform(t_lo, t_hi, B).astype(np.float32)
    esize = 2 if dt == dv.BF16 else 4
    ld = V if (V * esize) % 16 == 0 else (V + 16 // esize - 1) // (16 // esize) * (16 // esize)
    pad = (lambda x: np.pad(x, ((0, 0), (0, ld - V)))) if ld != V else (lambda x: x)
    out = dv.alloc_sampling_outputs(B, gamma, V, dt, DEV)
    say(f"weight sums seed={seed} V={V} dt={dt}")
    dv.dspark_accept_sampling(
        B, gamma, V, dt, logits_up(pad(c["tgt"]), dt), ld, c["tgt"].shape[0],
        up(np.asarray(c["cu"], np.int32)), logits_up(pad(c["drf"]), dt), ld,
        up(c["drafts"].reshape(B, gamma)), up(c["temps"]), up(_bits(c["ra"]).reshape(B, gamma)),
        up(_bits(c["rs"]).reshape(B, gamma + 1)), up(c["prefix"]), out)
    torch.cuda.synchronize()
    z = _slot_sums(out, B, gamma, V, dt)
    tgt = as_f32_rows(c["tgt"], "bf16" if dt == dv.BF16 else "f32")
    drf = as_f32_rows(c["drf"], "bf16" if dt == dv.BF16 else "f32")
    cu, checked, worst = c["cu"], 0, 0.0
    for r in range(B):
        l, T = int(cu[r + 1] - cu[r]), float(c["temps"][r])
        rows = [(r * (gamma + 1) + j, tgt[cu[r] + j]) for j in range(l)]
        rows += [(B * (gamma + 1) + r * gamma + k, drf[r * gamma + k]) for k in range(l - 1)]
        for slot, x in rows:
            ws = _exact_weights(x, T)
            want = float(np.sum(ws))
            bound = float(np.sum(F64.EPS_W * ws + 0.5 + 1e-5)) + 1e-9 * want
            assert abs(z[slot] - want) <= bound, (r, slot, T, z[slot], want, bound)
            worst = max(worst, abs(z[slot] - want) / want)
            checked += 1
    say(f"{checked} slot weight sums within the bound; largest relative error {worst:.3g}")


@pytest.mark.parametrize("V,dt", [(20000, dv.BF16), (6000, dv.F32), (3000, dv.BF16)])
def test_sampling_residual_near_equality(V, dt):
    """q equal to p except at one token d of tiny probability, whose q weight
    is e^5 times p's. The draft d is rejected (large accept words), and every
    other token has Wp Zq and Wq Zp within 2^-20 of each other (Zq - Zp is
    below 2^-20 Zp, checked on the kernels' own sums), so the residual sums and
    the draw decide membership on the exact path. With identical logits and
    maxima the residual is p's weight times Zq - Zp on every token but d, so
    the drawn token must be the inverse-CDF draw from p without d, within the
    band of a draw from p."""
    B, G = 8, 1
    rng = np.random.default_rng(V)
    temps = rng.uniform(0.7, 1.4, B).astype(np.float32)
    cu = np.arange(0, 2 * B + 1, 2, dtype=np.int32)
    rows = rng.normal(0, 2.5, (2 * B, V)).astype(np.float32)
    if dt == dv.BF16:
        rows = as_f32_rows(gen.f32_to_bf16_bits(rows), "bf16")
    drf = np.empty((B, V), np.float32)
    drafts = np.empty((B, G), np.int32)
    for r in range(B):
        p, T = rows[2 * r], float(temps[r])
        d = int(np.argmin(p))
        p[d] = p.max() - 18.5 * T  # a weight of about 20 units of 2^31
        q = p.copy()
        q[d] = p[d] + 5.0 * T
        if dt == dv.BF16:
            p[:] = as_f32_rows(gen.f32_to_bf16_bits(p[None]), "bf16")[0]
            q = as_f32_rows(gen.f32_to_bf16_bits(q[None]), "bf16")[0]
        drf[r] = q
        drafts[r, 0] = d
    ra = rng.integers(2**31, 2**32, (B, G), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, G + 1), dtype=np.uint64).astype(np.uint32)
    prefix = np.zeros(B, np.int32)
    tgt_in = gen.f32_to_bf16_bits(rows) if dt == dv.BF16 else rows
    drf_in = gen.f32_to_bf16_bits(drf) if dt == dv.BF16 else drf
    esize = 2 if dt == dv.BF16 else 4
    ld = V if (V * esize) % 16 == 0 else (V + 16 // esize - 1) // (16 // esize) * (16 // esize)
    pad = (lambda x: np.pad(x, ((0, 0), (0, ld - V)))) if ld != V else (lambda x: x)
    out = dv.alloc_sampling_outputs(B, G, V, dt, DEV)
    say(f"near equality V={V} dt={dt}")
    dv.dspark_accept_sampling(
        B, G, V, dt, logits_up(pad(tgt_in), dt), ld, 2 * B, up(cu), logits_up(pad(drf_in), dt), ld,
        up(drafts), up(temps), up(_bits(ra)), up(_bits(rs)), up(prefix), out)
    torch.cuda.synchronize()
    z = _slot_sums(out, B, G, V, dt)
    got = {"num_correct": out.num_correct.cpu().numpy(), "bonus": out.bonus.cpu().numpy(),
           "commit": out.commit_lens.cpu().numpy(), "new_seq": out.new_seq_lens.cpu().numpy(),
           "out_tokens": out.out_tokens.cpu().numpy(), "meta": out.accept_meta.cpu().numpy()}
    dtype = "bf16" if dt == dv.BF16 else "f32"
    check_f64(got, B, G, tgt_in, drf_in, dtype, cu, drafts, temps, ra, rs, prefix, tag="near")
    eps_p, eta_p = F64.prob_error_bound(V)
    for r in range(B):
        zp, zq = z[r * (G + 1)], z[B * (G + 1) + r * G]
        assert 0 < zq - zp < zp / 2**20, (r, zp, zq)  # the premise: every other token near
        assert got["num_correct"][r] == 0, r          # the draft is rejected
        w = F64.softmax64(rows[2 * r], float(temps[r]))
        w[drafts[r, 0]] = 0.0
        k, _, ok = F64._draw_check(w, F64.uniform(rs[r, 0]), int(got["bonus"][r]),
                                   eps_p + V * eta_p, V)
        assert ok and got["bonus"][r] != drafts[r, 0], (r, k, got["bonus"][r])
