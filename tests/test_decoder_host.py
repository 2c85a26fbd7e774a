"""The multi-round driver's protocol (the card's SpeculativeDecoder, sections
"Usage" and "API") on the CPU.  The verification step is the fp64 oracle,
through the decoder's test hook, so these tests check the host protocol (the
pending token, truncation, batching, the uniforms) against what the card
fixes: a greedy stream equals plain greedy target decoding, and a sampled
stream has the target's distribution."""
import numpy as np
import pytest
from scipy.stats import chi2

import oracle
from speculative_decoding_verification_row_amd import SpeculativeDecoder
from speculative_decoding_verification_row_amd.decoder import Governor

from _models import HashLM, TiedLM, greedy_decode, make_callbacks


def oracle_verify(greedy):
    """The oracle as the decoder's verification hook; it also returns every
    target row's argmax (the oracle's row statistics), which forcing rounds
    use."""
    def f(tp, dp, tk, u):
        o = oracle.verify_greedy(tp, tk) if greedy else oracle.verify_sample(tp, dp, tk, u)
        return o["n_accepted"], o["next_token"], o["stats"]["argmax"]
    return f


def _models(V, noise, sigma=2.0):
    target = HashLM(V, sigma=sigma, salt=11)
    return target, HashLM(V, salt=12, base=target, noise=noise)


@pytest.mark.parametrize("noise", [0.0, 1.0, 4.0])
@pytest.mark.parametrize("k", [0, 1, 4])
def test_greedy_stream_equals_plain_greedy_decoding(k, noise):
    target, draft = _models(50, noise)
    ds, ts = make_callbacks(target, draft, greedy=True)
    dec = SpeculativeDecoder(ds, ts, k=k, greedy=True, verify=oracle_verify(True))
    for prompt in ([1, 2, 3], [7], [0, 0, 0, 0]):
        assert dec.generate(prompt, max_new=23) == greedy_decode(target, prompt, 23)
    if k == 0:         # nothing proposed: one target token per round
        assert dec.stats.rounds == 3 * 23 and dec.stats.proposed == 0
    elif noise == 0.0:   # the draft is the target: every proposal is accepted
        assert dec.stats.accepted and all(a == k for a in dec.stats.accepted)
        assert dec.stats.acceptance_fraction() == 1.0
    else:
        assert dec.stats.rounds >= 3 * 23 // (k + 1)


def test_truncation_stop_token_and_batches():
    target, draft = _models(30, 2.0)
    for greedy in (True, False):
        ds, ts = make_callbacks(target, draft, greedy=greedy, seed=3)
        dec = SpeculativeDecoder(ds, ts, k=4, greedy=greedy, seed=5, verify=oracle_verify(greedy))
        for m in (0, 1, 2, 5, 6, 11):
            out = dec.generate([4, 5], max_new=m)
            assert len(out) == 2 + m and out[:2] == [4, 5]
        full = dec.generate([9], max_new=40)
        stop = full[5]
        ds, ts = make_callbacks(target, draft, greedy=greedy, seed=3)
        dec2 = SpeculativeDecoder(ds, ts, k=4, greedy=greedy, seed=5, verify=oracle_verify(greedy))
        if greedy:
            cut = dec2.generate([9], max_new=40, stop_token=stop)
            assert cut == full[:full.index(stop, 1) + 1]
    # batched callbacks: several prompts, each its own length
    ds, ts = make_callbacks(target, draft, greedy=True, batched=True)
    dec = SpeculativeDecoder(ds, ts, k=3, greedy=True, batched=True, verify=oracle_verify(True))
    prompts = [[1], [2, 3], [4, 5, 6]]
    outs = dec.generate(prompts, max_new=9)
    assert outs == [greedy_decode(target, p, 9) for p in prompts]


def test_sampled_streams_are_seeded():
    target, draft = _models(40, 1.5)
    res = []
    for _ in range(2):
        ds, ts = make_callbacks(target, draft, greedy=False, seed=8)
        dec = SpeculativeDecoder(ds, ts, k=4, greedy=False, seed=21, verify=oracle_verify(False))
        res.append(dec.generate([3, 1], max_new=30))
    assert res[0] == res[1]


def _joint_law(target, prompt, m, V):
    """Exact probability of every continuation of length m (V^m cells)."""
    law = {(): 1.0}
    for _ in range(m):
        nxt = {}
        for seq, w in law.items():
            p = target.row(list(prompt) + list(seq)).astype(np.float64)
            p /= p.sum()
            for x in range(V):
                nxt[seq + (x,)] = w * p[x]
        law = nxt
    return law


def sampled_law_check(verify, N=20000, V=4, k=3, m=3, seed=0, **dec_kw):
    """N sequences from one prompt, one batch: the empirical law of their
    first m tokens against the exact target law (chi-square, cells merged
    until each expects >= 10)."""
    target, draft = _models(V, 1.0, sigma=0.8)
    prompt = [2, 0, 1]
    ds, ts = make_callbacks(target, draft, greedy=False, seed=seed, batched=True)
    dec = SpeculativeDecoder(ds, ts, k=k, greedy=False, seed=seed + 1, batched=True, verify=verify, **dec_kw)
    outs = dec.generate([prompt] * N, max_new=m)
    law = _joint_law(target, prompt, m, V)
    keys = sorted(law)
    obs = {key: 0 for key in keys}
    for o in outs:
        obs[tuple(o[len(prompt):])] += 1
    exp = np.array([law[key] * N for key in keys])
    got = np.array([obs[key] for key in keys], np.float64)
    order = np.argsort(exp)
    e_cells, o_cells, ea, oa = [], [], 0.0, 0.0
    for j in order:
        ea += exp[j]
        oa += got[j]
        if ea >= 10:
            e_cells.append(ea)
            o_cells.append(oa)
            ea = oa = 0.0
    e_cells[-1] += ea
    o_cells[-1] += oa
    e_cells, o_cells = np.array(e_cells), np.array(o_cells)
    stat = float(((o_cells - e_cells) ** 2 / e_cells).sum())
    pval = float(chi2.sf(stat, len(e_cells) - 1))
    return pval, dec.stats


def test_sampled_stream_has_the_target_law():
    pval, stats = sampled_law_check(oracle_verify(False))
    assert pval > 1e-4, pval
    # the imperfect draft is both accepted and rejected
    h = stats.histogram(3)
    assert h[0] > 0 and h[3] > 0


# --------------------------------------------- telemetry and the governor --

def test_telemetry_counts_agree_with_the_rounds():
    target, draft = _models(40, 1.5)
    ds, ts = make_callbacks(target, draft, greedy=True)
    dec = SpeculativeDecoder(ds, ts, k=4, greedy=True, verify=oracle_verify(True))
    dec.generate([1, 2], max_new=200)
    st = dec.stats
    n = np.asarray(st.accepted)
    assert st.proposed == 4 * n.size and st.position_tested[0] == n.size
    for i in range(4):
        assert st.position_accepted[i] == int((n > i).sum())
        assert st.position_tested[i] == int((n >= i).sum())
    assert st.acceptance_fraction() == n.sum() / (4 * n.size)
    assert np.array_equal(st.histogram(4), np.bincount(n, minlength=5))
    # acceptance decays with the position only through the prefix rule
    assert np.all(st.position_rate() <= 1.0) and 0 < st.acceptance_fraction() < 1


@pytest.mark.parametrize("greedy", [True, False])
def test_governor_trips_on_a_zero_accept_round(greedy):
    target, draft = _models(40, 50.0)          # a draft that is almost always wrong
    ds, ts = make_callbacks(target, draft, greedy=greedy, seed=2)
    gov = Governor(alpha_threshold=0.0, window=4, trip_on_zero=True)
    dec = SpeculativeDecoder(ds, ts, k=4, greedy=greedy, seed=3, governor=gov, verify=oracle_verify(greedy))
    out = dec.generate([5], max_new=30)
    assert dec.stats.trips == 1 and dec.stats.ar_rounds > 0
    assert len(dec.stats.accepted) + dec.stats.ar_rounds == dec.stats.rounds
    if greedy:
        assert out == greedy_decode(target, [5], 30)
    # a new call drafts again
    dec.generate([6], max_new=10)
    assert dec.stats.trips == 2


def test_governor_threshold_and_perfect_draft():
    target, noisy = _models(40, 1.5)
    ds, ts = make_callbacks(target, noisy, greedy=True)
    dec = SpeculativeDecoder(ds, ts, k=4, greedy=True, verify=oracle_verify(True),
                             governor=Governor(alpha_threshold=0.95, window=2, trip_on_zero=False))
    assert dec.generate([1], max_new=60) == greedy_decode(target, [1], 60)
    assert dec.stats.trips == 1
    _, perfect = _models(40, 0.0)
    ds, ts = make_callbacks(target, perfect, greedy=True)
    dec = SpeculativeDecoder(ds, ts, k=4, greedy=True, verify=oracle_verify(True),
                             governor=Governor(alpha_threshold=0.95, window=2, trip_on_zero=True))
    dec.generate([1], max_new=60)
    assert dec.stats.trips == 0 and dec.stats.ar_rounds == 0


def test_governed_sampled_stream_keeps_the_target_law():
    pval, stats = sampled_law_check(oracle_verify(False), governor=Governor(alpha_threshold=0.7, window=1))
    assert pval > 1e-4, pval
    assert stats.trips > 1000 and stats.ar_rounds > 1000


def test_forced_acceptance():
    target, draft = _models(40, 2.0)
    for greedy in (True, False):
        ds, ts = make_callbacks(target, draft, greedy=greedy, seed=4)
        dec = SpeculativeDecoder(ds, ts, k=4, greedy=greedy, seed=6, verify=oracle_verify(greedy), forced_alpha=1.0)
        dec.generate([3], max_new=50)
        assert all(a == 4 for a in dec.stats.accepted) and dec.stats.rounds == 10
        # nothing forced in: every round emits the target's argmax, i.e. greedy decoding
        ds, ts = make_callbacks(target, draft, greedy=greedy, seed=4)
        dec = SpeculativeDecoder(ds, ts, k=4, greedy=greedy, seed=6, verify=oracle_verify(greedy), forced_alpha=0.0)
        assert dec.generate([3], max_new=20) == greedy_decode(target, [3], 20)
    ds, ts = make_callbacks(target, draft, greedy=True)
    dec = SpeculativeDecoder(ds, ts, k=4, greedy=True, verify=oracle_verify(True), forced_alpha=0.75)
    dec.generate([3], max_new=4000)
    want = sum(0.75 ** i for i in range(1, 5)) / 4      # E[leading successes] / k
    n = np.asarray(dec.stats.accepted)
    se = np.std(n) / np.sqrt(n.size) / 4
    assert abs(dec.stats.acceptance_fraction() - want) < 4 * se
    with pytest.raises(ValueError):
        SpeculativeDecoder(ds, ts, forced_alpha=1.5)
    # the forced token is the lowest-index argmax: with exact ties in every
    # target row, alpha = 0 is still plain greedy decoding (numpy.argmax)
    tied = TiedLM(40, sigma=2.0, salt=19)
    ds, ts = make_callbacks(tied, HashLM(40, salt=20, base=tied, noise=2.0), greedy=False, seed=2)
    dec = SpeculativeDecoder(ds, ts, k=3, greedy=False, seed=8, verify=oracle_verify(False), forced_alpha=0.0)
    assert dec.generate([5], max_new=25) == greedy_decode(tied, [5], 25)
    # a verify hook without the argmax is refused in a forcing round
    dec = SpeculativeDecoder(ds, ts, k=3, greedy=True, forced_alpha=0.5,
                             verify=lambda tp, dp, tk, u: oracle_verify(True)(tp, dp, tk, u)[:2])
    with pytest.raises(ValueError):
        dec.generate([5], max_new=5)
