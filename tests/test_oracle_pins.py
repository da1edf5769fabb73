"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself. Each test checks it against a
value a page prints, a hand derivation from the rule, a closed form, a
distributional identity checked by Monte Carlo, or an independent library
routine. The last group plants plausible mistakes in the oracle and checks that
the pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import specv_oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits(probs, T):
    with np.errstate(divide="ignore"):
        return T * np.log(np.asarray(probs, dtype=np.float64))


def _two_token_rows(p0, q0):
    """Draft and target rows over a 2-token vocabulary with P(token 0) = p0, q0."""
    return _logits([p0, 1.0 - p0], 1.0), _logits([q0, 1.0 - q0], 1.0)


def _monte_carlo_same_rows(p_row, q_row, N, n_trials, seed):
    """n_trials verifications whose N positions all use the same (p, q) rows.

    Draft tokens are drawn from p by the input generator's Gumbel-max sampler;
    the oracle is then run on every trial. Returns the oracle results.
    """
    rng = np.random.default_rng(seed)
    draft = np.tile(p_row, (N, 1))
    target = np.tile(q_row, (N + 1, 1))
    tokens = np.stack([synth.gumbel_max_tokens(np.broadcast_to(p_row, (n_trials, p_row.size)), 1.0, rng)
                       for _ in range(N)], axis=1)
    ua = synth.grid_uniforms(rng, (n_trials, N)).astype(np.float64)
    us = synth.grid_uniforms(rng, (n_trials,)).astype(np.float64)
    return oracle.verify_trials(draft, target, tokens, ua, us, 1.0)


# ---------------------------------------------------------------- page values

def test_worked_acceptance_example():
    """Draft prob 0.9 vs verifier prob 0.45 is accepted with probability 0.5 (thakicloud guide)."""
    g = _load("page_values.json")["worked_acceptance"]
    p_row, q_row = _two_token_rows(g["draft_prob"], g["target_prob"])
    # Exact threshold: accepted for u just below 0.5, rejected at 0.5 (strict test).
    for u, accepted in ((0.5 - 2 ** -24, True), (0.5, False), (0.0, True), (0.75, False)):
        r = oracle.verify_sequence(p_row[None], np.stack([q_row, q_row]), [0], [u], 0.3, 1.0)
        assert (r.n_accepted == 1) == accepted, u
    # Frequency over 10^5 uniforms.
    rng = np.random.default_rng(11)
    n = 100_000
    u = synth.grid_uniforms(rng, (n, 1)).astype(np.float64)
    res = oracle.verify_trials(p_row[None], np.stack([q_row, q_row]), np.zeros((n, 1), np.int32), u,
                               np.full(n, 0.5), 1.0)
    freq = np.mean([r.n_accepted == 1 for r in res])
    sigma = math.sqrt(0.25 / n)
    assert abs(freq - g["acceptance_probability"]) < 4 * sigma
    # After the rejection the residual is (q - p)_+ = [0, 0.45]: token 1 always.
    assert all(r.tokens[0] == 1 for r in res if r.n_accepted == 0)


def test_all_accepted_gives_n_plus_one_tokens():
    """p == q accepts every draft: N = 5 gives 6 tokens (lesson, Step 3)."""
    g = _load("page_values.json")["all_accepted_tokens"]
    N = g["n_draft"]
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(vocab=500)
    b = synth.make_batch(wl, seed=3)
    t64 = synth.widen(b.target_logits[0], b.dtype)
    rng = np.random.default_rng(5)
    for trial in range(50):
        tokens = synth.gumbel_max_tokens(t64[:N], 1.0, rng)
        ua = synth.grid_uniforms(rng, (N,)).astype(np.float64)
        r = oracle.verify_sequence(t64[:N], t64, tokens, ua, float(rng.random()), 1.0)
        assert r.n_accepted == N
        emitted = sum(t >= 0 for t in r.tokens)
        assert emitted == g["tokens_emitted"]


def test_target_at_least_draft_always_accepts_and_bounds():
    """q(d) >= p(d) always accepts; 1 <= emitted <= N+1 (tech.blogsailing post, section 3)."""
    g = _load("page_values.json")["emitted_bounds"]
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(batch=6, vocab=700)
    b = synth.make_batch(wl, seed=9)
    d64 = synth.widen(b.draft_logits, b.dtype)
    t64 = synth.widen(b.target_logits, b.dtype)
    N = wl.n_draft
    checked = 0
    for s in range(wl.batch):
        q = special.softmax(t64[s], axis=-1)
        p = special.softmax(d64[s], axis=-1)
        for u in (0.0, 0.5, 1.0 - 2 ** -24):
            r = oracle.verify_sequence(d64[s], t64[s], b.draft_tokens[s], np.full(N, u),
                                       float(b.sample_uniforms[s]), 1.0)
            emitted = sum(t >= 0 for t in r.tokens)
            assert g["min_emitted"] <= emitted <= N + g["max_emitted_minus_k"]
            for i in range(N):
                d = b.draft_tokens[s, i]
                if i < r.n_accepted:
                    continue
                if i == r.n_accepted and r.n_accepted < N:
                    assert q[i, d] < p[i, d] * (1 + 1e-12), "rejected a token the verifier likes more"
                    checked += 1
                break
    assert checked > 0


@pytest.mark.parametrize("case", _load("hand_examples.json")["cases"], ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    T = case["temperature"]
    draft = _logits(case["draft_probs"], T)
    target = _logits(case["target_probs"], T)
    ua = np.asarray(case["accept_uniforms"], dtype=np.float32).astype(np.float64)
    us = float(np.float32(case["sample_uniform"]))
    r = oracle.verify_sequence(draft, target, case["draft_tokens"], ua, us, T)
    assert r.n_accepted == case["n_accepted"]
    assert r.tokens == case["tokens"]


@pytest.mark.parametrize("case", _load("hand_examples.json")["greedy_cases"], ids=lambda c: c["name"])
def test_greedy_hand_cases(case):
    target = np.asarray(case["target_logits"], dtype=np.float64)
    N = len(case["draft_tokens"])
    draft = np.zeros((N, target.shape[1]))
    r = oracle.verify_sequence(draft, target, case["draft_tokens"], np.zeros(N), 0.5, 0.0)
    assert r.n_accepted == case["n_accepted"]
    assert r.tokens == case["tokens"]
    assert r.lse is None and r.sample_margin is None


# ------------------------------------------------------- closed forms (rates)

def _tau(alpha, N):
    return (1 - alpha ** (N + 1)) / (1 - alpha)


def test_page_closed_form_values():
    """The printed figures follow from tau = (1 - a^(N+1)) / (1 - a) and survival a^k."""
    g = _load("page_values.json")["tokens_per_verify"]
    rt = g["rule_of_thumb"]
    assert abs(_tau(rt["alpha"], rt["n_draft"]) - rt["about"]) <= rt["band"]
    for k, pct in enumerate(g["survival_percent"], start=1):
        assert round(100 * g["survival_alpha"] ** k) == pct
    ten = g["ten_drafts"]
    assert ten["range"][0] <= _tau(ten["alpha"], ten["n_draft"]) <= ten["range"][1]
    flat = g["flat_at_040"]
    assert abs(_tau(flat["alpha"], flat["n_large"]) - _tau(flat["alpha"], flat["n_small"])) < flat["max_difference"]


@pytest.mark.parametrize("p0,q0,N", [(0.9, 0.65, 5), (0.9, 0.6, 4), (0.7, 0.1, 3)])
def test_geometric_law_monte_carlo(p0, q0, N):
    """Same (p, q) at every position: P(n >= k) = a^k, E[emitted] = tau(a, N), a = sum min(p, q)."""
    alpha = min(p0, q0) + min(1 - p0, 1 - q0)
    p_row, q_row = _two_token_rows(p0, q0)
    n = 60_000
    res = _monte_carlo_same_rows(p_row, q_row, N, n, seed=int(1000 * p0 + 100 * q0 + N))
    nacc = np.array([r.n_accepted for r in res])
    for k in range(1, N + 1):
        f = np.mean(nacc >= k)
        a_k = alpha ** k
        assert abs(f - a_k) < 4 * math.sqrt(a_k * (1 - a_k) / n) + 1e-12, (k, f, a_k)
    emitted = nacc + 1
    tau = _tau(alpha, N)
    assert abs(emitted.mean() - tau) < 4 * emitted.std() / math.sqrt(n)


def test_page_survival_percentages_by_monte_carlo():
    """At a = 0.7 the survival of draft k is 70/49/34/24 percent (thakicloud guide)."""
    g = _load("page_values.json")["tokens_per_verify"]
    p_row, q_row = _two_token_rows(0.8, 0.5)  # sum min(p, q) = 0.5 + 0.2 = 0.7
    n = 100_000
    res = _monte_carlo_same_rows(p_row, q_row, 4, n, seed=77)
    nacc = np.array([r.n_accepted for r in res])
    for k, pct in enumerate(g["survival_percent"], start=1):
        f = np.mean(nacc >= k)
        assert abs(100 * f - pct) < 0.5 + 400 * math.sqrt(f * (1 - f) / n)


# ----------------------------------------- distribution equivalence (chi-square)

def _tiny_trials(n, seed=0, temperature=None):
    wl = synth.workload("tiny_b1_n4_v16_f32")
    tr = synth.make_trials(wl, seed, n)
    T = float(tr.temperature[0])
    d64 = synth.widen(tr.draft_logits[0], tr.dtype)
    t64 = synth.widen(tr.target_logits[0], tr.dtype)
    res = oracle.verify_trials(d64, t64, tr.draft_tokens, tr.accept_uniforms.astype(np.float64),
                               tr.sample_uniforms.astype(np.float64), T)
    return d64, t64, T, tr, res


def _position_pvalues(t64, d64, T, res):
    """Chi-square p-values: the token emitted at position i (given i is reached) vs q_i.

    q_i comes from scipy's softmax, independently of the oracle.
    """
    q = special.softmax(t64 / T, axis=-1)
    p = special.softmax(d64 / T, axis=-1)
    N = d64.shape[0]
    nacc = np.array([r.n_accepted for r in res])
    toks = np.array([r.tokens for r in res])
    pvals, accept_z = [], []
    for i in range(N + 1):
        reached = nacc >= i
        counts = np.bincount(toks[reached, i], minlength=q.shape[1])
        expected = reached.sum() * q[i]
        pvals.append(stats.chisquare(counts, expected).pvalue)
        if i < N:
            alpha = np.minimum(p[i], q[i]).sum()
            acc = (nacc[reached] > i).mean()
            accept_z.append((acc - alpha) / math.sqrt(alpha * (1 - alpha) / reached.sum()))
    return pvals, accept_z


@pytest.fixture(scope="module")
def tiny_mc():
    return _tiny_trials(100_000, seed=0)


def test_emitted_tokens_follow_verifier(tiny_mc):
    """Every emitted token, and the bonus, follows q (lesson Step 5; 10^5 trials)."""
    d64, t64, T, _, res = tiny_mc
    pvals, _ = _position_pvalues(t64, d64, T, res)
    assert min(pvals) > 1e-3, pvals


def test_acceptance_rate_is_sum_min(tiny_mc):
    """P(accept at i | reached i) = sum_x min(p_i, q_i) within 4 sigma."""
    d64, t64, T, _, res = tiny_mc
    _, z = _position_pvalues(t64, d64, T, res)
    assert max(abs(v) for v in z) < 4.0, z


def test_residual_draw_follows_normalised_residual(tiny_mc):
    """Conditioned on a rejection at i, the drawn token follows (q_i - p_i)_+ / S."""
    d64, t64, T, _, res = tiny_mc
    q = special.softmax(t64 / T, axis=-1)
    p = special.softmax(d64 / T, axis=-1)
    nacc = np.array([r.n_accepted for r in res])
    toks = np.array([r.tokens for r in res])
    for i in range(d64.shape[0]):
        sel = nacc == i
        r = np.clip(q[i] - p[i], 0, None)
        r = r / r.sum()
        counts = np.bincount(toks[sel, i], minlength=q.shape[1])
        support = r > 0
        assert counts[~support].sum() == 0, "drew a token with zero residual weight"
        assert stats.chisquare(counts[support], sel.sum() * r[support]).pvalue > 1e-3


def test_tempered_equivalence():
    """At T = 0.7 the emitted tokens follow softmax(z_target / 0.7)."""
    wl = synth.workload("tiny_b1_n4_v16_f32")
    base = synth.make_batch(wl, seed=4)
    d64 = synth.widen(base.draft_logits[0], base.dtype)
    t64 = synth.widen(base.target_logits[0], base.dtype)
    T = float(np.float32(0.7))
    rng = np.random.default_rng(21)
    n, N = 60_000, wl.n_draft
    tokens = np.stack([synth.gumbel_max_tokens(np.broadcast_to(d64[i], (n, d64.shape[1])), T, rng)
                       for i in range(N)], axis=1)
    res = oracle.verify_trials(d64, t64, tokens, synth.grid_uniforms(rng, (n, N)).astype(np.float64),
                               synth.grid_uniforms(rng, (n,)).astype(np.float64), T)
    pvals, z = _position_pvalues(t64, d64, T, res)
    assert min(pvals) > 1e-3, pvals
    assert max(abs(v) for v in z) < 4.0


def test_greedy_limit_emits_argmax():
    """T = 0 is the low-temperature limit: the emitted token is the target argmax."""
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(batch=8, vocab=2000)
    b = synth.make_batch(wl, seed=12)
    d64 = synth.widen(b.draft_logits, b.dtype)
    t64 = synth.widen(b.target_logits, b.dtype)
    for s in range(wl.batch):
        g = oracle.verify_sequence(d64[s], t64[s], np.argmax(d64[s], axis=-1), np.zeros(5), 0.5, 0.0)
        cold = oracle.verify_sequence(d64[s], t64[s], np.argmax(d64[s], axis=-1), np.full(5, 0.5),
                                      0.5, 1e-5)
        assert g.n_accepted == cold.n_accepted
        assert g.tokens == cold.tokens


# ---------------------------------------------------- library special cases

def test_log_normaliser_matches_scipy_and_mpmath():
    wl = synth.workload("b64_n5_v128256_bf16").with_sizes(batch=2, vocab=32000)
    b = synth.make_batch(wl, seed=1)
    T = float(b.temperature[0])
    rows = synth.widen(b.target_logits[0], b.dtype)
    L = oracle.tempered_log_normaliser(rows, T)
    ref = special.logsumexp(rows / T, axis=-1)
    assert np.max(np.abs(L - ref) / np.maximum(1.0, np.abs(ref))) < 1e-13
    import mpmath
    mpmath.mp.dps = 50
    row = rows[1, :3000]
    exact = mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(float(z)) / mpmath.mpf(T)) for z in row))
    assert abs(float(oracle.tempered_log_normaliser(row[None], T)[0]) - float(exact)) < 1e-12 * abs(float(exact))


def _cdf_pin_holds(cdf) -> bool:
    """Brute force at V = 16: over a fine grid of u, token k is drawn for a
    fraction w_k / S of the grid, zero-weight tokens never, monotone in u, and
    u*S exactly on C_{k-1} draws k."""
    rng = np.random.default_rng(2)
    for trial in range(5):
        w = rng.random(16)
        w[rng.random(16) < 0.3] = 0.0
        w[0] = 0.0
        w[3] = 0.0
        grid = np.arange(1 << 14) / float(1 << 14)
        drawn = np.array([cdf(w, u)[0] for u in grid])
        if not np.all(np.diff(drawn) >= 0) or not np.all(w[drawn] > 0):
            return False
        freq = np.bincount(drawn, minlength=16) / grid.size
        if np.max(np.abs(freq - w / w.sum())) > 2.0 / grid.size:
            return False
        C = np.cumsum(w)
        for k in np.nonzero(w)[0]:
            lo = C[k - 1] if k > 0 else 0.0
            u = lo / C[-1]
            if u * C[-1] == lo and u < 1.0 and cdf(w, u)[0] != k:
                return False
    return True


def test_inverse_cdf_brute_force():
    assert _cdf_pin_holds(oracle.inverse_cdf)


def test_greedy_first_argmax_with_ties():
    row = np.array([0.0, 2.0, -1.0, 2.0, 2.0])
    assert oracle.first_argmax(row) == 1
    assert oracle.first_argmax(np.array([-np.inf, -np.inf, 3.0])) == 2


def test_invalid_inputs_give_sentinel():
    draft = np.zeros((2, 4))
    target = np.zeros((3, 4))
    for T, toks in ((float("nan"), [0, 1]), (-1.0, [0, 1]), (float("inf"), [0, 1]), (-0.5, [0, 1]),
                    (1.0, [0, 4]), (1.0, [-1, 0]), (0.0, [7, 0])):
        r = oracle.verify_sequence(draft, target, toks, [0.5, 0.5], 0.5, T)
        assert r.n_accepted == -1 and r.tokens == [-1, -1, -1]


def test_every_finite_positive_temperature_is_computed():
    """Tiny temperatures are inside the rule's domain: as T -> 0 the tempered
    distributions tend to point masses, so away from ties the result is the
    greedy one (the oracle's fp64 keeps z / T finite down to the smallest
    float32 T)."""
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(batch=6, vocab=3000)
    b = synth.make_batch(wl, seed=31)
    d64 = synth.widen(b.draft_logits, b.dtype)
    t64 = synth.widen(b.target_logits, b.dtype)
    for T in (2.0 ** -61, 1e-30, float(np.float32(2.0 ** -149))):
        for s in range(wl.batch):
            toks = np.argmax(d64[s], axis=-1)
            g = oracle.verify_sequence(d64[s], t64[s], toks, np.full(5, 0.5), 0.5, 0.0)
            r = oracle.verify_sequence(d64[s], t64[s], toks, np.full(5, 0.5), 0.5, T)
            assert r.n_accepted >= 0 and all(np.isfinite(r.lse))
            assert (r.n_accepted, r.tokens) == (g.n_accepted, g.tokens), (T, s)
    # A ratio beyond the fp64 range (q(d) > p(d) at a tiny T) exceeds every uniform: accepted.
    d = np.array([[1.0, 0.0]])
    t = np.array([[0.0, 1.0], [0.0, 1.0]])
    r = oracle.verify_sequence(d, t, [1], [1.0 - 2 ** -24], 0.5, 1e-30)
    assert r.n_accepted == 1 and r.tokens == [1, 1]


# ------------------------------------------------------ planted mistakes

def _pins_fail(monkeypatch, attr, bad):
    monkeypatch.setattr(specv_oracle, attr, bad)
    d64, t64, T, _, res = _tiny_trials(30_000, seed=5)
    pvals, z = _position_pvalues(t64, d64, T, res)
    return min(pvals) < 1e-6 or max(abs(v) for v in z) > 6.0


def test_planted_residual_mistake_is_caught(monkeypatch):
    assert _pins_fail(monkeypatch, "residual_weights", lambda q, p: q)


def test_planted_ratio_inversion_is_caught(monkeypatch):
    assert _pins_fail(monkeypatch, "acceptance_ratio", lambda lq, lp: math.exp(lp - lq))


def test_planted_bonus_mistake_is_caught(monkeypatch):
    flat = lambda q: np.ones_like(q)  # noqa: E731
    assert _pins_fail(monkeypatch, "bonus_weights", flat)


def test_planted_cdf_mistake_is_caught():
    def cdf_ge(w, u):  # '>=' instead of '>': zero-weight tokens can be drawn
        C = np.cumsum(w)
        k = int(np.nonzero(C >= u * C[-1])[0][0])
        return k, 0.0, float(C[-1])

    def cdf_shifted(w, u):  # off by one: the token after the crossing
        k = oracle.inverse_cdf(w, u)[0]
        return min(k + 1, len(w) - 1), 0.0, 0.0

    assert not _cdf_pin_holds(cdf_ge)
    assert not _cdf_pin_holds(cdf_shifted)


def test_planted_temperature_mistake_is_caught(monkeypatch):
    case = [c for c in _load("hand_examples.json")["cases"] if c["name"] == "temperature_two"][0]
    orig = specv_oracle.tempered_log_normaliser
    monkeypatch.setattr(specv_oracle, "tempered_log_normaliser", lambda z, T: orig(z, 1.0))
    T = case["temperature"]
    r = oracle.verify_sequence(_logits(case["draft_probs"], T), _logits(case["target_probs"], T),
                               case["draft_tokens"], np.asarray(case["accept_uniforms"]),
                               case["sample_uniform"], T)
    assert (r.n_accepted, r.tokens) != (case["n_accepted"], case["tokens"])


# ------------------------------------------------------------ margins

def _hand_result(case):
    T = case["temperature"]
    ua = np.asarray(case["accept_uniforms"], dtype=np.float32).astype(np.float64)
    us = float(np.float32(case["sample_uniform"]))
    return oracle.verify_sequence(_logits(case["draft_probs"], T), _logits(case["target_probs"], T),
                                  case["draft_tokens"], ua, us, T)


def _hand_margins_hold() -> bool:
    for case in _load("hand_examples.json")["cases"]:
        r = _hand_result(case)
        want = [float(m) for m in case["decision_margins"]]
        if len(r.decision_margins) != len(want):
            return False
        for got, w in zip(r.decision_margins, want):
            if math.isinf(w):
                if not math.isinf(got):
                    return False
            elif not abs(got - w) <= 2e-7:
                return False
        if not abs(r.sample_margin - case["sample_margin"]) <= 2e-7:
            return False
    return True


def _brute_force_margins_hold(seed=3) -> bool:
    """V = 16 brute force: the draw margin is the distance from u*S to the
    nearest CDF edge (every edge 0, C_0, ..., C_15 examined), and each decision
    margin is |u_i - r_i| with r_i = q_i(d_i)/p_i(d_i) from scipy's softmax."""
    rng = np.random.default_rng(seed)
    for trial in range(200):
        w = rng.random(16)
        w[rng.random(16) < 0.3] = 0.0
        if w.sum() == 0:
            continue
        u = float(synth.grid_uniforms(rng, ()))
        k, margin, S = oracle.inverse_cdf(w, u)
        edges = np.concatenate([[0.0], np.cumsum(w)])
        if not abs(margin - np.min(np.abs(u * S - edges))) <= 1e-15:
            return False
    for trial in range(60):
        N, V = 4, 16
        d = rng.normal(size=(N, V))
        t = np.concatenate([d, rng.normal(size=(1, V))]) + rng.normal(scale=1.5, size=(N + 1, V))
        T = float(np.float32(rng.choice([0.5, 1.0, 2.0])))
        p = special.softmax(d / T, axis=-1)
        q = special.softmax(t / T, axis=-1)
        toks = np.array([rng.choice(V, p=p[i]) for i in range(N)])
        ua = synth.grid_uniforms(rng, (N,)).astype(np.float64)
        r = oracle.verify_sequence(d, t, toks, ua, 0.5, T)
        tested = min(r.n_accepted + 1, N)
        if len(r.decision_margins) != tested:
            return False
        for i in range(tested):
            want = abs(ua[i] - q[i, toks[i]] / p[i, toks[i]])
            if not abs(r.decision_margins[i] - want) <= 1e-12 * max(1.0, want):
                return False
    return True


def test_margins_of_hand_cases():
    assert _hand_margins_hold()


def test_margins_by_brute_force():
    assert _brute_force_margins_hold()


@pytest.mark.parametrize("attr,bad", [
    ("decision_margin", lambda u, r: 0.0),                          # no margin at all
    ("decision_margin", lambda u, r: abs(u - 1.0 / r) if r else math.inf),  # inverted ratio
    ("cdf_margin", lambda t, lo, up: 0.0),
    ("cdf_margin", lambda t, lo, up: abs(up - t)),                  # upper edge only
    ("cdf_margin", lambda t, lo, up: abs(t - lo)),                  # lower edge only
])
def test_planted_margin_mistakes_are_caught(monkeypatch, attr, bad):
    monkeypatch.setattr(specv_oracle, attr, bad)
    assert not (_hand_margins_hold() and _brute_force_margins_hold())


# ------------------------------------------------------- draft-side sampler

def _sampler_frequencies_hold(T, n=100_000, seed=8) -> bool:
    wl = synth.workload("tiny_b1_n4_v16_f32")
    b = synth.make_batch(wl, seed=2)
    z = synth.widen(b.draft_logits[0, 0], b.dtype)
    rng = np.random.default_rng(seed)
    us = synth.grid_uniforms(rng, (n,)).astype(np.float64)
    toks = np.array([oracle.sample_row(z, T, u).token for u in us])
    q = special.softmax(z / T)
    return stats.chisquare(np.bincount(toks, minlength=z.size), n * q).pvalue > 1e-3


@pytest.mark.parametrize("T", [1.0, float(np.float32(0.7)), 2.5])
def test_sampler_follows_tempered_softmax(T):
    """Drawn tokens follow softmax(z / T) (chi-square against scipy's softmax)."""
    assert _sampler_frequencies_hold(T)


def test_sampler_brute_force_cdf():
    """V = 16: over a fine grid of u the token is the smallest k with C_k > u*S,
    each token drawn for a share q_k of the grid, monotone in u."""
    rng = np.random.default_rng(4)
    for trial in range(5):
        z = rng.normal(scale=2.0, size=16)
        z[rng.random(16) < 0.2] = -np.inf
        z[5] = 1.0
        q = special.softmax(z)
        grid = np.arange(1 << 13) / float(1 << 13)
        drawn = np.array([oracle.sample_row(z, 1.0, u).token for u in grid])
        assert np.all(np.diff(drawn) >= 0) and np.all(q[drawn] > 0)
        freq = np.bincount(drawn, minlength=16) / grid.size
        assert np.max(np.abs(freq - q)) <= 2.0 / grid.size + 1e-12


def test_sampler_greedy_and_invalid():
    row = np.array([0.0, 2.0, -1.0, 2.0])
    assert oracle.sample_row(row, 0.0, 0.9).token == 1
    for T in (float("nan"), -1.0, float("inf")):
        assert oracle.sample_row(row, T, 0.5).token == -1
    # Tiny T tends to the argmax.
    assert oracle.sample_row(np.array([0.0, 2.0, 1.999]), 1e-30, 0.99).token == 1


def test_planted_sampler_temperature_mistake_is_caught(monkeypatch):
    orig = specv_oracle.tempered_probabilities
    monkeypatch.setattr(specv_oracle, "tempered_probabilities", lambda z, T: orig(z, 1.0))  # T dropped
    assert not _sampler_frequencies_hold(2.5)


# ------------------------------------------------------- acceptance telemetry

@pytest.mark.parametrize("case", _load("hand_examples.json")["acceptance_rate_cases"], ids=lambda c: c["name"])
def test_acceptance_rates_hand_cases(case):
    T = case["temperature"]
    alpha, tau = oracle.acceptance_rates(_logits(case["draft_probs"], T), _logits(case["target_probs"], T),
                                         case["draft_tokens"], T)
    assert np.allclose(alpha, case["alpha"], rtol=0, atol=1e-12)
    assert abs(tau - case["tau"]) < 1e-12


@pytest.mark.parametrize("case", _load("hand_examples.json")["greedy_acceptance_cases"], ids=lambda c: c["name"])
def test_acceptance_rates_greedy(case):
    target = np.asarray(case["target_logits"])
    N = len(case["draft_tokens"])
    alpha, tau = oracle.acceptance_rates(np.zeros((N, target.shape[1])), target, case["draft_tokens"], 0.0)
    assert alpha == case["alpha"] and tau == case["tau"]


def test_tau_closed_form_and_page_values():
    """Constant alpha at every position: tau = (1 - a^(N+1)) / (1 - a) (lesson);
    the page's rule of thumb a = 0.75, N = 5 gives about 3, and a = 0.7 with
    ten drafts leaves 3 to 4 tokens per pass (guide)."""
    g = _load("page_values.json")["tokens_per_verify"]
    for a, N in ((0.75, 5), (0.7, 10), (0.4, 3), (0.4, 7), (0.9, 16)):
        p0, q0 = 0.95, 0.95 - (1.0 - a)  # sum min(p, q) = q0 + (1 - p0) = a
        d = np.tile(_logits([p0, 1 - p0], 1.0), (N, 1))
        t = np.tile(_logits([q0, 1 - q0], 1.0), (N + 1, 1))
        alpha, tau = oracle.acceptance_rates(d, t, np.zeros(N, int), 1.0)
        assert np.allclose(alpha, a, atol=1e-12)
        assert abs(tau - (1 - a ** (N + 1)) / (1 - a)) < 1e-12
    rt = g["rule_of_thumb"]
    d = np.tile(_logits([0.95, 0.05], 1.0), (rt["n_draft"], 1))
    t = np.tile(_logits([0.7, 0.3], 1.0), (rt["n_draft"] + 1, 1))
    assert abs(oracle.acceptance_rates(d, t, np.zeros(rt["n_draft"], int), 1.0)[1] - rt["about"]) <= rt["band"]


def test_acceptance_rate_is_the_monte_carlo_frequency(tiny_mc):
    """alpha_i from the formula against the oracle's own accept decisions over
    10^5 trials (the acceptance rule and sum min(p, q) are two independent
    routes to the same number), and alpha_i = 1 - sum_x (q_i - p_i)_+."""
    d64, t64, T, tr, res = tiny_mc
    alpha, tau = oracle.acceptance_rates(d64, t64, tr.draft_tokens[0], T)
    nacc = np.array([r.n_accepted for r in res])
    q = special.softmax(t64 / T, axis=-1)
    p = special.softmax(d64 / T, axis=-1)
    for i in range(d64.shape[0]):
        reached = nacc >= i
        f = (nacc[reached] > i).mean()
        a = alpha[i]
        assert abs(f - a) < 4 * math.sqrt(a * (1 - a) / reached.sum())
        assert abs(a - (1.0 - np.clip(q[i] - p[i], 0, None).sum())) < 1e-12
    emitted = nacc + 1
    assert abs(emitted.mean() - tau) < 4 * emitted.std() / math.sqrt(len(res))


def test_planted_acceptance_mistake_is_caught(monkeypatch):
    case = [c for c in _load("hand_examples.json")["acceptance_rate_cases"] if c["name"] == "temperature_two"][0]
    T = case["temperature"]
    orig = specv_oracle.tempered_probabilities
    monkeypatch.setattr(specv_oracle, "tempered_probabilities", lambda z, T: orig(z, 1.0))  # T dropped
    alpha, _ = oracle.acceptance_rates(_logits(case["draft_probs"], T), _logits(case["target_probs"], T),
                                       case["draft_tokens"], T)
    assert not np.allclose(alpha, case["alpha"], atol=1e-6)


# ------------------------------------------------------- KV-cache commit

def _kv_exercise_holds(commit) -> bool:
    g = _load("kv_rollback_exercise.json")
    P, E, L = 4, 6, 32
    N, prefix = g["n_draft"], g["prefix_len"]
    rng = np.random.default_rng(9)
    cache = rng.integers(0, 256, size=(P, 1, L, E), dtype=np.uint8)
    scratch = rng.integers(0, 256, size=(P, 1, N, E), dtype=np.uint8)
    n_acc = g["rejected_position_counting_from_1"] - 1
    if n_acc != g["n_accepted"]:
        return False
    new, new_len = commit(cache, np.array([prefix]), scratch, np.array([n_acc]))
    if int(new_len[0]) != g["expected_len"]:
        return False
    want = []
    for kind, idx in zip(g["expected_read"][0::2], g["expected_read"][1::2]):
        want.append(cache[:, 0, idx, :] if kind == "prefix" else scratch[:, 0, idx, :])
    read = new[:, 0, :int(new_len[0]), :]
    return np.array_equal(read, np.stack(want, axis=1)) and np.array_equal(new[:, 0, int(new_len[0]):], cache[:, 0, int(new_len[0]):])


def test_kv_rollback_exercise():
    """The lesson's exercise 4: a 10-token prefix, 5 drafts, rejection at the
    third; the next read is the prefix plus the first 2 drafts, exactly."""
    assert _kv_exercise_holds(oracle.kv_commit)


def test_kv_commit_edge_cases():
    rng = np.random.default_rng(10)
    P, B, L, N, E = 2, 6, 12, 5, 8
    cache = rng.integers(0, 256, size=(P, B, L, E), dtype=np.uint8)
    scratch = rng.integers(0, 256, size=(P, B, N, E), dtype=np.uint8)
    lens = np.array([0, 3, 7, 9, 2, 12])
    nacc = np.array([0, 5, 5, 4, -1, 1])   # nothing, all, exactly full, overflow, invalid, overflow
    new, nl = oracle.kv_commit(cache, lens, scratch, nacc)
    assert nl.tolist() == [0, 8, 12, -1, -1, -1]
    assert np.array_equal(new[:, 0], cache[:, 0])
    assert np.array_equal(new[:, 1, 3:8], scratch[:, 1, :5]) and np.array_equal(new[:, 1, :3], cache[:, 1, :3])
    assert np.array_equal(new[:, 2, 7:12], scratch[:, 2])
    for b in (3, 4, 5):
        assert np.array_equal(new[:, b], cache[:, b])
    assert np.array_equal(new[:, 1, 8:], cache[:, 1, 8:])


def test_planted_kv_mistakes_are_caught():
    def keeps_rejected(cache, lens, scratch, nacc):  # commits the rejected draft too
        return oracle.kv_commit(cache, lens, scratch, np.minimum(np.asarray(nacc) + 1, scratch.shape[2]))

    def wrong_offset(cache, lens, scratch, nacc):  # overwrites the prefix's last entry
        return oracle.kv_commit(cache, np.asarray(lens) - 1, scratch, nacc)

    assert not _kv_exercise_holds(keeps_rejected)
    assert not _kv_exercise_holds(wrong_offset)
