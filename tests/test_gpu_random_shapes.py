"""GPU parity on seeded random shapes: B, K and V drawn at random (V
log-uniform up to 70000, so one to eighteen 4096-value chunks with ragged
tails; K = 0 for every eighth), greedy, sampled and logits, statistics on and
off, the sampled and logits form (walks or one block per row) left to the
library or forced, in turn.  Every
sequence is compared with the fp64 oracle to the bars of the other parity
tests: greedy bit for bit, sampled and logits identical outside the 1e-5
boundary band."""
import numpy as np
import pytest
import torch

import oracle
from oracle.logits import verify_sample_logits
import speculative_decoding_verification_row_amd as sv

from _parity import BAND_PROB, check_greedy, check_logits, check_sampled, compare_outputs
from _forms import set_form

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_SHAPES = 64


def _case(msg):
    print(f"\n[gpu case] {msg}", flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    sv.load_library()
    yield
    torch.cuda.synchronize()


def _shape(j):
    """B up to 64, K up to 12, V log-uniform over [2, 70000] (half the shapes
    over [10000, 70000]), the whole batch kept under 3e7 values so that the
    oracle finishes in a second or two."""
    rng = np.random.default_rng(9000 + j)
    B = int(rng.integers(1, 65))
    K = 0 if j % 8 == 7 else int(rng.integers(1, 13))
    lo = np.log(10000.0) if j % 4 < 2 else np.log(2.0)
    V = int(np.exp(rng.uniform(lo, np.log(70000.0))))
    while B > 1 and B * (2 * K + 1) * V > 3e7:
        B //= 2
    return B, K, V, rng


# every third shape leaves the sampled form to the library's size rule (which
# picks one block per row at these sizes); the others force walks or rows
FORMS = ("auto", "walks", "rows")


def _rows(rng, B, K, V):
    """Unnormalised rows with zeros and tied maxima; draft tokens from q
    half the time, else the target's argmax or a random token."""
    p = rng.random((B, K + 1, V)).astype(np.float32) * rng.uniform(0.5, 2.0, (B, K + 1, 1)).astype(np.float32)
    q = rng.random((B, K, V)).astype(np.float32)
    p[rng.random(p.shape) < 0.15] = 0
    p[..., 0] += np.float32(1e-3)
    q[..., -1] += np.float32(1e-3)
    for b in range(B):
        for i in range(K + 1):
            p[b, i, rng.choice(V, size=min(V, 2), replace=False)] = p[b, i].max()
    t = np.empty((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            r = rng.random()
            if r < 0.5:
                c = np.cumsum(q[b, i].astype(np.float64))
                t[b, i] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), V - 1)
            elif r < 0.8:
                t[b, i] = int(np.argmax(p[b, i]))
            else:
                t[b, i] = int(rng.integers(0, V))
    u = rng.random((B, K + 1), dtype=np.float32)
    return p, q, t, u


def _dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


@pytest.mark.parametrize("j", range(N_SHAPES))
def test_random_shape(j, monkeypatch):
    B, K, V, rng = _shape(j)
    stats = bool(j % 2)
    form = FORMS[j % 3]
    if form != "auto":
        set_form(monkeypatch, form)
    _case(f"random shape {j}: B={B} K={K} V={V} stats={stats} sampled form={form}")
    p, q, t, u = _rows(rng, B, K, V)
    tp, dp, dt, ud = _dev(p, q, t, u)

    r = sv.sv_verify_greedy_batched(tp, dt, stats=stats or None)
    torch.cuda.synchronize()
    check_greedy(r[0].cpu().numpy(), r[1].cpu().numpy(),
                 sv.stats_to_numpy(r[2]) if stats else None, oracle.verify_greedy(p, t))

    r = sv.sv_verify_sample_batched(tp, dp, dt, ud, stats=stats or None)
    torch.cuda.synchronize()
    check_sampled(r[0].cpu().numpy(), r[1].cpu().numpy(),
                  sv.stats_to_numpy(r[2]) if stats else None, oracle.verify_sample(p, q, t, u))

    # the same rows read as logits (their log, with -1e4 for zeros), one temperature
    tau = float(rng.choice([0.7, 1.0, 1.6]))
    lp = np.where(p > 0, np.log(np.maximum(p, 1e-30)), -1e4).astype(np.float32)
    lq = np.where(q > 0, np.log(np.maximum(q, 1e-30)), -1e4).astype(np.float32)
    tl, dl = _dev(lp, lq)
    n, nx = sv.sv_verify_sample_logits_batched(tl, dl, dt, ud, tau)
    torch.cuda.synchronize()
    check_logits(n.cpu().numpy(), nx.cpu().numpy(), verify_sample_logits(lp, lq, t, u, tau))


def _shape_wide(j):
    """Shapes the first set does not reach: large batches over small V (the
    library's own rule then picks walks), long drafts (K up to 32), and
    every third shape's rows at a 4- but not 16-byte aligned address."""
    rng = np.random.default_rng(19000 + j)
    if j % 2 == 0:
        B = int(rng.integers(300, 900))
        K = int(rng.integers(1, 5))
        V = int(rng.integers(2, 4097))
    else:
        B = int(rng.integers(1, 9))
        K = int(rng.integers(8, 33))
        V = int(np.exp(rng.uniform(np.log(2.0), np.log(40000.0))))
    while B > 1 and B * (2 * K + 1) * V > 3e7:
        B //= 2
    return B, K, V, j % 3 == 2, rng


def _dev_offset(a):
    """A copy of `a` on the device, one float past a 16-byte boundary."""
    flat = np.ascontiguousarray(a).reshape(-1)
    buf = torch.zeros(flat.size + 1, dtype=torch.float32, device=DEV)
    buf[1:].copy_(torch.from_numpy(flat))
    return buf[1:].view(a.shape)


@pytest.mark.parametrize("j", range(N_SHAPES))
def test_random_shape_wide(j):
    B, K, V, unaligned, rng = _shape_wide(j)
    stats = bool(j % 4 == 1)
    _case(f"random wide shape {j}: B={B} K={K} V={V} unaligned={unaligned} stats={stats}")
    p, q, t, u = _rows(rng, B, K, V)
    dt, ud = _dev(t, u)
    if unaligned:
        tp, dp = _dev_offset(p), _dev_offset(q)
    else:
        tp, dp = _dev(p, q)

    r = sv.sv_verify_greedy_batched(tp, dt, stats=stats or None)
    torch.cuda.synchronize()
    check_greedy(r[0].cpu().numpy(), r[1].cpu().numpy(),
                 sv.stats_to_numpy(r[2]) if stats else None, oracle.verify_greedy(p, t))

    r = sv.sv_verify_sample_batched(tp, dp, dt, ud, stats=stats or None)
    torch.cuda.synchronize()
    check_sampled(r[0].cpu().numpy(), r[1].cpu().numpy(),
                  sv.stats_to_numpy(r[2]) if stats else None, oracle.verify_sample(p, q, t, u))

    tau = float(rng.choice([0.8, 1.0, 1.3]))
    lp = np.where(p > 0, np.log(np.maximum(p, 1e-30)), -1e4).astype(np.float32)
    lq = np.where(q > 0, np.log(np.maximum(q, 1e-30)), -1e4).astype(np.float32)
    tl, dl = (_dev_offset(lp), _dev_offset(lq)) if unaligned else _dev(lp, lq)
    n, nx = sv.sv_verify_sample_logits_batched(tl, dl, dt, ud, tau)
    torch.cuda.synchronize()
    check_logits(n.cpu().numpy(), nx.cpu().numpy(), verify_sample_logits(lp, lq, t, u, tau))


def test_layout_churn_across_tag_wrap():
    """300 calls on one workspace, cycling through five shapes and the three
    entry points, so that every call reads over words that calls of other
    layouts and kinds left behind, and the tags wrap around once: every
    output stays the oracle's (each shape's inputs are the same every time
    it comes round)."""
    _case("layout churn: 300 calls on one workspace across the tag wrap")
    shapes = [(3, 4, 5000), (40, 2, 326), (7, 9, 9000), (1, 1, 70001), (64, 3, 1500)]
    cases = []
    need = 0
    for s, (B, K, V) in enumerate(shapes):
        rng = np.random.default_rng(31000 + s)
        p, q, t, u = _rows(rng, B, K, V)
        lp = np.where(p > 0, np.log(np.maximum(p, 1e-30)), -1e4).astype(np.float32)
        lq = np.where(q > 0, np.log(np.maximum(q, 1e-30)), -1e4).astype(np.float32)
        og, os_, ol = oracle.verify_greedy(p, t), oracle.verify_sample(p, q, t, u), verify_sample_logits(lp, lq, t, u, 1.0)
        cases.append(((B, K, V), _dev(p, q, t, u, lp, lq), og, os_, ol))
        need = max(need, sv.sv_workspace_size(B, K, V, True))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    for j in range(300):
        (B, K, V), (tp, dp, dt, ud, tl, dl), og, os_, ol = cases[j % len(cases)]
        kind = (j // len(cases)) % 3
        if kind == 0:
            n, nx = sv.sv_verify_greedy_batched(tp, dt, workspace=ws)
            ref = og
        elif kind == 1:
            n, nx = sv.sv_verify_sample_batched(tp, dp, dt, ud, workspace=ws)
            ref = os_
        else:
            n, nx = sv.sv_verify_sample_logits_batched(tl, dl, dt, ud, 1.0, workspace=ws)
            ref = ol
        torch.cuda.synchronize()
        n, nx = n.cpu().numpy(), nx.cpu().numpy()
        if kind == 0:
            assert np.array_equal(n, ref["n_accepted"]) and np.array_equal(nx, ref["next_token"]), (j, B, K, V)
        elif kind == 1:
            compare_outputs(n, nx, ref, BAND_PROB)
        else:
            check_logits(n, nx, ref)
    assert sv.sv_workspace_error(ws) == 0
