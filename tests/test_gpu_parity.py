"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case prints its name before touching the GPU.  Sizes: small and ragged
shapes spanning several 8192-value chunks and a ragged tail (the oracle checks
every sequence), then the five workloads at full size in the launch
configuration the benchmark times (the oracle checks every sequence, or a
seeded sample of 128 for the 1024-sequence workload, plus properties that hold
for all).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.device import device_batch
import speculative_decoding_verification_row_amd as sv

from _parity import BAND_PROB, FP64_RTOL, check_greedy, check_sampled
from _forms import FORMS, set_form

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[gpu case] {msg}", flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    sv.load_library()
    yield
    torch.cuda.synchronize()


def _to_dev(*arrays):
    return [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def _outs(r, stats):
    """numpy outputs of a verify call; stats None when none were requested."""
    torch.cuda.synchronize()
    if stats:
        n, nx, st = r
        return n.cpu().numpy(), nx.cpu().numpy(), sv.stats_to_numpy(st)
    n, nx = r
    return n.cpu().numpy(), nx.cpu().numpy(), None


def run_greedy(tp, dt, stats=True, **kw):
    tpd, dtd = _to_dev(tp, dt)
    return _outs(sv.sv_verify_greedy_batched(tpd, dtd, stats=stats or None, **kw), stats)


def run_sample(tp, dp, dt, u, stats=True, **kw):
    tpd, dpd, dtd, ud = _to_dev(tp, dp, dt, u)
    return _outs(sv.sv_verify_sample_batched(tpd, dpd, dtd, ud, stats=stats or None, **kw), stats)


def _random_rows(rng, B, K, V, ties=True, zeros=True):
    p = rng.random((B, K + 1, V)).astype(np.float32)
    q = rng.random((B, K, V)).astype(np.float32)
    if zeros:
        p[rng.random(p.shape) < 0.2] = 0
        q[rng.random(q.shape) < 0.2] = 0
        p[..., 0] += np.float32(1e-3)
        q[..., -1] += np.float32(1e-3)
    if ties:
        for b in range(B):
            for i in range(K + 1):
                idx = rng.choice(V, size=min(V, 3), replace=False)
                p[b, i, idx] = p[b, i].max()
    t = np.empty((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            r = rng.random()
            t[b, i] = np.argmax(p[b, i]) if r < 0.5 else rng.integers(0, V)
    u = rng.random((B, K + 1), dtype=np.float32)
    return p, q, t, u


# ----------------------------------------------------------- small shapes --

SMALL = [(1, 0, 1), (3, 0, 7), (2, 1, 2), (4, 2, 3), (5, 4, 1000), (3, 3, 1003), (2, 2, 8192),
         (2, 3, 8193), (2, 2, 16389), (3, 4, 32000), (2, 5, 40001), (1, 2, 65536 + 4),
         (3, 9, 5000), (2, 17, 9000)]   # the last two: K + 1 rows in 3 and 5 groups of the finishing combine


# Both kernel variants: with row statistics, and without (the configuration
# the benchmark times, whose finishing work differs).
STATS = [True, False]


# Both forms of the sampled pass: walks down the draft rows, and one block per
# draft row (which the library picks by itself when every block fits on the
# chip at once).
@pytest.fixture(params=FORMS)
def form(request, monkeypatch):
    set_form(monkeypatch, request.param)
    return request.param


@pytest.mark.parametrize("stats", STATS, ids=["stats", "nostats"])
@pytest.mark.parametrize("B,K,V", SMALL, ids=lambda x: str(x))
def test_greedy_small(B, K, V, stats):
    _case(f"greedy small B={B} K={K} V={V} stats={stats}")
    rng = np.random.default_rng(B * 1000 + K * 100 + V)
    p, _, t, _ = _random_rows(rng, B, K, V)
    n, nx, st = run_greedy(p, t, stats=stats)
    check_greedy(n, nx, st, oracle.verify_greedy(p, t))


@pytest.mark.parametrize("stats", STATS, ids=["stats", "nostats"])
@pytest.mark.parametrize("B,K,V", SMALL, ids=lambda x: str(x))
def test_sampled_small(B, K, V, stats, form):
    _case(f"sampled small B={B} K={K} V={V} stats={stats} form={form}")
    rng = np.random.default_rng(7 + B * 1000 + K * 100 + V)
    p, q, t, u = _random_rows(rng, B, K, V)
    n, nx, st = run_sample(p, q, t, u, stats=stats)
    check_sampled(n, nx, st, oracle.verify_sample(p, q, t, u))


@pytest.mark.parametrize("stats", STATS, ids=["stats", "nostats"])
@pytest.mark.parametrize("family,B,K,V", [("c1", 16, 4, 32000), ("c3", 24, 5, 24577),
                                          ("c4", 32, 8, 12000), ("c5", 6, 16, 30011)])
def test_sampled_families_reduced(family, B, K, V, stats, form):
    _case(f"sampled {family} B={B} K={K} V={V} stats={stats} form={form}")
    b = workloads.make_batch(family, B, K, V, seed=5)
    args = (b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    n, nx, st = run_sample(*args, stats=stats)
    rep = check_sampled(n, nx, st, oracle.verify_sample(*args))
    print(f"  parity {rep}")


# ------------------------------------------------------------ workloads --

def _gpu_outputs(db, sampled, stats=True):
    if sampled:
        r = sv.sv_verify_sample_batched(db["tp"], db["dp"], db["dt"], db["u"], stats=stats or None)
    else:
        r = sv.sv_verify_greedy_batched(db["tp"], db["dt"], stats=stats or None)
    return _outs(r, stats)


def _oracle_on(c, rows, sampled, seed=0):
    b = workloads.make_batch(c["family"], c["B"], c["K"], c["V"], seed=seed, seqs=rows)
    if sampled:
        return oracle.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms,
                                    threads=workloads.default_workers()), b
    return oracle.verify_greedy(b.target_probs, b.draft_tokens, threads=workloads.default_workers()), b


@pytest.mark.parametrize("cfg,mode", [(2, "greedy"), (3, "sampled"), (5, "greedy"), (5, "sampled"),
                                      (4, "sampled")])
def test_workload_full_size(cfg, mode):
    c = dict(workloads.CONFIGS[cfg])
    sampled = mode == "sampled"
    _case(f"workload {cfg} {mode} B={c['B']} K={c['K']} V={c['V']} (generating)")
    db = device_batch(c["family"], c["B"], c["K"], c["V"], seed=0, device=DEV, sampled=sampled)
    _case(f"workload {cfg} {mode}: running, with row statistics and without (the benchmark's launch)")
    # the cached workspace these calls use, cleared so that only they can set
    # its recompute flag (earlier tests force recomputes on purpose)
    B, K, V = c["B"], c["K"], c["V"]
    ws = sv.workspace_for(B, K, V, sampled, DEV)
    sv.sv_workspace_init(ws)
    n, nx, st = _gpu_outputs(db, sampled)
    n0, nx0, _ = _gpu_outputs(db, sampled, stats=False)
    assert np.all((n >= 0) & (n <= K)) and np.all((nx >= 0) & (nx < V))
    # both variants take every decision from the same words: identical outputs
    assert np.array_equal(n0, n) and np.array_equal(nx0, nx)
    rows = None
    if B > 256:
        rows = np.sort(np.random.default_rng(cfg).choice(B, size=128, replace=False))
    orc, hb = _oracle_on(c, rows, sampled)
    if sampled:
        rep = check_sampled(n, nx, st, orc, rows=rows)
        check_sampled(n0, nx0, None, orc, rows=rows)
        print(f"  parity {rep}")
        if cfg == 4:
            qeqp = np.array([d["q_equals_p"] for d in db["info"]])
            assert qeqp.sum() == B // 4
            assert np.all(n[qeqp] == K)            # q = p accepts every draft
    else:
        check_greedy(n, nx, st, orc, rows=rows)
        check_greedy(n0, nx0, None, orc, rows=rows)
        if cfg == 2:
            m = np.array([d["m"] for d in db["info"]])
            assert np.array_equal(n, m)
    assert sv.sv_workspace_error(ws) == 0
    assert _slow_path_flag(ws) == 0   # siblings were co-scheduled: nothing recomputed
    del db
    torch.cuda.empty_cache()


def test_workload1_600_rounds_and_law():
    """Workload 1 as the card measures it: 600 seeded rounds of B=1, one call
    per round, greedy and sampled; every round against the oracle, and the
    GPU's mean accepted length against the analytic law."""
    _case("workload 1: 600 rounds, greedy + sampled")
    ns, means, vars_, bnd = [], [], [], 0
    for r in range(600):
        b = workloads.make_config(1, rnd=r)
        args = (b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
        n, nx, st = run_sample(*args)
        orc = oracle.verify_sample(*args)
        bnd += check_sampled(n, nx, st, orc)["boundary"]
        gn, gx, gst = run_greedy(b.target_probs, b.draft_tokens)
        check_greedy(gn, gx, gst, oracle.verify_greedy(b.target_probs, b.draft_tokens))
        m, v = oracle.expected_accepted_length(orc["alpha"][0])
        ns.append(int(n[0]))
        means.append(m)
        vars_.append(v)
    se = np.sqrt(np.sum(vars_)) / 600
    print(f"  mean n {np.mean(ns):.4f} analytic {np.mean(means):.4f} se {se:.4f} boundary {bnd}")
    assert abs(np.mean(ns) - np.mean(means)) <= 3 * se


# ---------------------------------------------------------- enumeration --

def test_exact_enumeration_cells_on_gpu(form):
    """Every cell of the tiny-V enumeration (one sequence each) as one batch:
    the GPU must return the oracle's outcome for every cell (cells are far
    from their boundaries)."""
    from test_oracle_law import _cells, _instance
    for K, V, seed in [(0, 8, 1), (1, 5, 3), (2, 6, 6), (3, 8, 8)]:
        _case(f"enumeration K={K} V={V} form={form}")
        p, q = _instance(np.random.default_rng(1000 + seed), K, V)
        t, u, wts, expect = _cells(p, q)
        B = len(wts)
        tp = np.broadcast_to(p, (B, K + 1, V)).copy()
        dp = np.broadcast_to(q, (B, K, V)).copy()
        n, nx, st = run_sample(tp, dp, t, u)
        got = list(zip(n.tolist(), nx.tolist()))
        assert got == expect
        check_sampled(n, nx, st, oracle.verify_sample(tp, dp, t, u))


# ----------------------------------------------------------- edge cases --

def test_edge_empty_batch():
    _case("edge: B=0")
    tp = torch.empty((0, 3, 100), dtype=torch.float32, device=DEV)
    n, nx = sv.sv_verify_greedy_batched(tp, torch.empty((0, 2), dtype=torch.int32, device=DEV))
    assert n.numel() == 0 and nx.numel() == 0
    n, nx = sv.sv_verify_sample_batched(tp, torch.empty((0, 2, 100), dtype=torch.float32, device=DEV),
                                        torch.empty((0, 2), dtype=torch.int32, device=DEV),
                                        torch.empty((0, 3), dtype=torch.float32, device=DEV))
    assert n.numel() == 0


def test_edge_out_of_range_tokens_and_one_hot(form):
    _case(f"edge: out-of-range tokens, one-hot rows, q = p, form={form}")
    rng = np.random.default_rng(11)
    B, K, V = 8, 3, 9000
    p, q, t, u = _random_rows(rng, B, K, V, ties=False)
    t[0, 0] = -1
    t[1, 1] = V
    t[2, 2] = 2**31 - 1
    p[3] = 0
    p[3, np.arange(K + 1), [5, 8191, 8192, 8999]] = 1.5      # one-hot, across chunk edges
    q[4] = p[4, :K]                                          # q = p: every draft accepted
    t[4] = [np.argmax(p[4, i]) for i in range(K)]
    u[4, :K] = np.float32(1) - np.float32(2**-24)
    n, nx, st = run_sample(p, q, t, u)
    check_sampled(n, nx, st, oracle.verify_sample(p, q, t, u))
    assert n[0] == 0 and n[4] == K
    gn, gx, gst = run_greedy(p, t)
    check_greedy(gn, gx, gst, oracle.verify_greedy(p, t))


def test_edge_extreme_scales(form):
    """The method is scale-free (the test compares u q(t) P with p(t) Q, the
    residual is p Q - q P): rows scaled far from 1 decide as the oracle does
    on the same f32 values.  Subnormal rows (every value below 2^-126, so
    the loads, maxima and sums see subnormal f32), rows near 2^110, and a
    target and draft 2^200 apart; statistics to the usual bar."""
    _case(f"edge: extreme scales (subnormal to 2^110), form={form}")
    rng = np.random.default_rng(23)
    B, K, V = 8, 3, 9000
    p, q, t, u = _random_rows(rng, B, K, V, ties=True)
    scales = [(2.0**-140, 2.0**-140), (2.0**100, 2.0**-100), (2.0**-130, 1.0), (2.0**110, 2.0**110),
              (1.0, 2.0**-135), (2.0**-100, 2.0**100)]
    for b, (sp, sq) in enumerate(scales):
        p[b] *= np.float32(sp)
        q[b] *= np.float32(sq)
    assert p[0].max() < np.finfo(np.float32).tiny and p[0].max() > 0 and np.isfinite(p).all()
    n, nx, st = run_sample(p, q, t, u)
    check_sampled(n, nx, st, oracle.verify_sample(p, q, t, u))
    gn, gx, gst = run_greedy(p, t)
    check_greedy(gn, gx, gst, oracle.verify_greedy(p, t))


def test_edge_all_equal_rows_tie_to_index_zero():
    _case("edge: constant rows")
    B, K, V = 3, 2, 20000
    p = np.full((B, K + 1, V), 0.25, np.float32)
    t = np.zeros((B, K), np.int32)
    t[1, 0] = 1
    n, nx, st = run_greedy(p, t)
    assert list(n) == [2, 0, 2] and list(nx) == [0, 0, 0]
    assert np.all(st["argmax"] == 0)


def test_edge_max_vocabulary():
    _case(f"edge: V = SV_MAX_V = 524288")
    rng = np.random.default_rng(12)
    B, K, V = 2, 2, 524288
    p, q, t, u = _random_rows(rng, B, K, V, ties=True, zeros=False)
    n, nx, st = run_sample(p, q, t, u)
    check_sampled(n, nx, st, oracle.verify_sample(p, q, t, u))
    gn, gx, gst = run_greedy(p, t)
    check_greedy(gn, gx, gst, oracle.verify_greedy(p, t))


@pytest.mark.parametrize("B,K,V", [(2, 4096, 5), (2, 257, 9000)], ids=lambda x: str(x))
def test_edge_max_draft_length(B, K, V, form):
    """K = SV_MAX_K draft rows (and a long K over two chunks): one sequence
    with random rows, one whose drafts are all accepted (q = p, t = argmax,
    u just below 1), so the bonus draw follows the last of K rows."""
    _case(f"edge: long draft B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(K + V)
    p, q, t, u = _random_rows(rng, B, K, V, ties=True, zeros=True)
    q[1] = p[1, :K]
    t[1] = np.argmax(p[1, :K], axis=1)
    u[1, :K] = np.float32(1) - np.float32(2**-24)
    os_, og = oracle.verify_sample(p, q, t, u), oracle.verify_greedy(p, t)
    assert os_["n_accepted"][1] == K and og["n_accepted"][1] == K
    for stats in STATS:
        check_sampled(*run_sample(p, q, t, u, stats=stats), os_)
        check_greedy(*run_greedy(p, t, stats=stats), og)


def test_edge_unaligned_rows_use_scalar_path(form):
    """A base pointer that is 4- but not 16-byte aligned selects the scalar
    load path; results must not change."""
    _case(f"edge: unaligned base pointers, form={form}")
    rng = np.random.default_rng(13)
    B, K, V = 3, 3, 20000
    p, q, t, u = _random_rows(rng, B, K, V)
    big_p = torch.zeros(B * (K + 1) * V + 1, dtype=torch.float32, device=DEV)
    big_q = torch.zeros(B * K * V + 1, dtype=torch.float32, device=DEV)
    tpd = big_p[1:].view(B, K + 1, V)
    dpd = big_q[1:].view(B, K, V)
    tpd.copy_(torch.from_numpy(p))
    dpd.copy_(torch.from_numpy(q))
    dtd, ud = _to_dev(t, u)
    os_, og = oracle.verify_sample(p, q, t, u), oracle.verify_greedy(p, t)
    for stats in STATS:
        check_sampled(*_outs(sv.sv_verify_sample_batched(tpd, dpd, dtd, ud, stats=stats or None), stats), os_)
        check_greedy(*_outs(sv.sv_verify_greedy_batched(tpd, dtd, stats=stats or None), stats), og)


# ------------------------------------------ determinism and B-invariance --

def test_determinism_and_batch_invariance():
    _case("determinism: run twice; sequence alone vs in batch; greedy vs sampled p-row stats")
    b = workloads.make_batch("c3", 48, 5, 40000, seed=17)
    args = (b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    r1 = run_sample(*args)
    r2 = run_sample(*args)
    for x, y in zip(r1, r2):
        assert x.tobytes() == y.tobytes()
    for s in (0, 17, 47):
        one = run_sample(*(a[s:s + 1] for a in args))
        assert one[2].tobytes() == r1[2][s:s + 1].tobytes()
        assert int(one[0][0]) == int(r1[0][s]) and int(one[1][0]) == int(r1[1][s])
    # greedy and sampled cut rows into different chunk sizes, so their fp64
    # masses agree to rounding only; argmax and max value are exact in both
    g = run_greedy(b.target_probs, b.draft_tokens)
    for f in ("argmax", "max_p"):
        assert g[2][f].tobytes() == r1[2][f].tobytes()
    rel = np.abs(g[2]["sum_p"] - r1[2]["sum_p"]) / r1[2]["sum_p"]
    assert float(rel.max()) <= FP64_RTOL


def test_workspace_reuse_across_sizes_and_streams():
    _case("workspace: shrinking/growing sizes, explicit workspace, side stream")
    rng = np.random.default_rng(19)
    ws = torch.empty(sv.sv_workspace_size(16, 6, 70000, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    for B, K, V in [(16, 6, 70000), (3, 2, 9000), (9, 6, 17), (16, 6, 70000)]:
        p, q, t, u = _random_rows(rng, B, K, V)
        n, nx, st = run_sample(p, q, t, u, workspace=ws)
        check_sampled(n, nx, st, oracle.verify_sample(p, q, t, u))
        gn, gx, gst = run_greedy(p, t, workspace=ws)
        check_greedy(gn, gx, gst, oracle.verify_greedy(p, t))
    assert sv.sv_workspace_error(ws) == 0
    s = torch.cuda.Stream()
    p, q, t, u = _random_rows(rng, 4, 3, 30000)
    tpd, dpd, dtd, ud = _to_dev(p, q, t, u)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        n, nx = sv.sv_verify_sample_batched(tpd, dpd, dtd, ud)
    s.synchronize()
    orc = oracle.verify_sample(p, q, t, u)
    check_sampled(n.cpu().numpy(), nx.cpu().numpy(), None, orc)


def _slow_path_flag(ws):
    torch.cuda.synchronize()
    return int(ws[4:8].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("B,K,V", [(6, 5, 40000), (3, 0, 9000), (4, 3, 10001), (2, 9, 70001)],
                         ids=lambda x: str(x))
def test_recompute_path_is_bit_identical(B, K, V, form, monkeypatch):
    """Readers that recompute a sibling's partial (the path taken when a
    sibling has not been scheduled within the wait bound) produce exactly the
    published values: forcing every reader to recompute changes no bit."""
    _case(f"recompute path B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(B * 1000 + K * 10 + V % 7)
    p, q, t, u = _random_rows(rng, B, K, V)
    ref_s = run_sample(p, q, t, u)
    ref_g = run_greedy(p, t)
    ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    assert _slow_path_flag(ws) == 0
    monkeypatch.setenv("SV_VERIFY_FORCE_RECOMPUTE", "1")
    got_s = run_sample(p, q, t, u, workspace=ws)
    got_g = run_greedy(p, t, workspace=ws)
    monkeypatch.delenv("SV_VERIFY_FORCE_RECOMPUTE")
    assert _slow_path_flag(ws) == 1
    for x, y in zip(ref_s, got_s):
        assert x.tobytes() == y.tobytes()
    for x, y in zip(ref_g, got_g):
        assert x.tobytes() == y.tobytes()
    check_sampled(*got_s, oracle.verify_sample(p, q, t, u))
    check_greedy(*got_g, oracle.verify_greedy(p, t))


def test_workspace_tags_wrap_around():
    """Each call tags the words it publishes; after 255 calls the tags start
    over on a cleared workspace.  A large call, 260 small ones on the same
    workspace, then the large one again: every result is unchanged."""
    _case("workspace tag wrap-around: 262 calls on one workspace")
    rng = np.random.default_rng(23)
    big = _random_rows(rng, 8, 5, 30000)
    small = _random_rows(rng, 2, 1, 5000)
    ws = torch.empty(sv.sv_workspace_size(8, 5, 30000, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    first_big = run_sample(*big, workspace=ws)
    first_small = None
    dev_small = _to_dev(*small)
    for j in range(260):
        n, nx = sv.sv_verify_sample_batched(*dev_small, workspace=ws)
        cur = (n.cpu().numpy(), nx.cpu().numpy())
        if first_small is None:
            first_small = cur
        assert all(x.tobytes() == y.tobytes() for x, y in zip(cur, first_small)), j
    again = run_sample(*big, workspace=ws)
    for x, y in zip(first_big, again):
        assert x.tobytes() == y.tobytes()
    check_sampled(*again, oracle.verify_sample(*big))
    assert _slow_path_flag(ws) == 0


def test_binding_and_abi_errors():
    _case("argument errors through the binding")
    tp = torch.rand((2, 3, 100), device=DEV)
    dt = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        sv.sv_verify_greedy_batched(tp.double(), dt)
    with pytest.raises(ValueError):
        sv.sv_verify_greedy_batched(tp, dt[:, :1].contiguous())
    with pytest.raises(ValueError):
        sv.sv_verify_greedy_batched(tp.cpu(), dt)
    with pytest.raises(ValueError):   # a strided view: the kernels read rows by pointer
        sv.sv_verify_greedy_batched(torch.rand((2, 3, 200), device=DEV)[:, :, ::2], dt)
    with pytest.raises(ValueError):
        sv.sv_verify_greedy_batched(tp, dt, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        sv.sv_verify_greedy_batched(tp, dt, n_accepted=torch.zeros(3, dtype=torch.int32, device=DEV))
    with pytest.raises(TypeError):
        sv.sv_verify_sample_batched(tp, tp[:, :2].contiguous(), dt, torch.rand((2, 3), device=DEV).double())
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(sv.SVError) as e:
        sv.sv_verify_greedy_batched(tp, dt, workspace=small)
    assert e.value.status == -2
    big = torch.rand((1, 2, 524289), device=DEV)
    with pytest.raises(sv.SVError) as e:
        sv.sv_verify_greedy_batched(big, torch.zeros((1, 1), dtype=torch.int32, device=DEV))
    assert e.value.status == -4


def test_card_usage_single_sequence():
    """The card's call shape: target_probs [K+1, V], draft_tokens [K]."""
    _case("card usage: 2-D inputs")
    b = workloads.make_batch("c1", 1, 4, 32000, seed=23)
    tp = torch.from_numpy(b.target_probs[0]).to(DEV)
    dt = torch.from_numpy(b.draft_tokens[0]).to(DEV)
    n, nx = sv.verify_greedy(tp, dt)
    o = oracle.verify_greedy(b.target_probs, b.draft_tokens)
    assert (n, nx) == (int(o["n_accepted"][0]), int(o["next_token"][0]))
    dp = torch.from_numpy(b.draft_probs[0]).to(DEV)
    u = torch.from_numpy(b.uniforms[0]).to(DEV)
    n, nx = sv.verify_sample(tp, dp, dt, u)
    o = oracle.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    assert n == int(o["n_accepted"][0])
    if not (o["diag"]["draw_margin"][0] <= BAND_PROB):
        assert nx == int(o["next_token"][0])
