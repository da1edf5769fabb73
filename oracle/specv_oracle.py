"""Oracle: plain, slow fp64 CPU speculative-sampling verification.

TEST INFRASTRUCTURE ONLY. The test-suite, the package smoke check and the CPU
baseline leg of the benchmark are the only callers. The HIP library never
imports or calls this module, and this module imports nothing from it.

Pages cited (titles as published; sections named as on the page):

* LESSON: "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com,
  speculative-decoding lesson).
* BLOG: "LLM 추론 지연을 2배 이상 단축하는 투기적 디코딩(Speculative Decoding)과
  검증 샘플링 아키텍처" (tech.blogsailing.com).
* GUIDE: "친구가 먼저 쓰고 선생님이 채점합니다: 투기 디코딩 쉽게 읽기"
  (thakicloud.com). GUIDE names the draft distribution q and the target p; here,
  as in LESSON, q is the verifier (target) and p the draft.

What is computed, per sequence with temperature T, draft rows i = 0..N-1 and
verifier rows i = 0..N (LESSON "핵심 알고리즘(Core algorithm)", steps 2-6):

1. p_i = softmax(z^draft_i / T), q_i = softmax(z^target_i / T), through the
   per-row log-normaliser L = log sum_x exp(z_x / T).
2. Left to right, draft token d_i is accepted with probability
   min(1, q_i(d_i) / p_i(d_i)): accept iff u_i < q_i(d_i) / p_i(d_i) (LESSON
   "Step 1: 거절 단계", BLOG section 3 verification loop, GUIDE "답이 바뀌지
   않는다는 보장"). A zero draft probability accepts (LESSON Step 1 treats the
   ratio as infinite).
3. At the first rejection j a replacement is drawn from the normalised residual
   (q_j - p_j)_+ (LESSON step 5 and "Step 2: 잔차 분포"); if all N are accepted
   a bonus token is drawn from q_N (LESSON step 6).
4. Temperature 0 is the greedy limit: d_i is accepted iff it is the first argmax
   of target row i, and the emitted token is the first argmax of target row j.

Readings where the pages are silent (each also listed in the design notes):

* The categorical draw that the pages call but never define is an inverse CDF
  in ascending token order: the token is the smallest k with
  C_k > u * S, C_k = sum_{x<=k} w_x, S = C_{V-1}; should rounding leave no such
  k, the last token with positive weight is taken.
* If the residual sums to zero (only possible through rounding) the draw falls
  back to q_j.
* One accept uniform per position (u_i) and one sample uniform per sequence are
  passed in; the accept test is strict.
* The temperature domain is T = 0 (greedy) or any finite T > 0; a negative,
  NaN or infinite T marks the sequence invalid (n_accepted = -1, all tokens
  -1), as do draft tokens outside [0, V). With float32 logits (|z| < 2^128)
  and a float32 T >= 2^-149, z / T stays finite in fp64, so every such T is
  computed exactly as written.
* Decision margins, the distance of a float decision from its boundary, are
  recorded so that a parity check can tell rounding ties from real errors:
  |u_i - q_i(d_i)/p_i(d_i)| for each accept test made (decision_margin), and
  the distance from u*S to the nearer edge of the chosen token's CDF interval
  [C_{k-1}, C_k), in probability-mass units (cdf_margin).

Beyond the verification itself (the steps around it on the pages):

* sample_row: the draft-side draw of a token from softmax(z / T) (lesson,
  "핵심 알고리즘(Core algorithm)" step 2 and Step 3's draft loop), by the same
  inverse CDF; T = 0 takes the first argmax.
* acceptance_rates: the per-position acceptance probability
  alpha_i = sum_x min(p_i(x), q_i(x)) and the expected tokens per verifier
  pass tau = sum_{k=0..N} prod_{i<k} alpha_i (lesson, "속도 향상을 결정하는 것";
  guide, "몇 글자를 미리 쓰게 할까요").
* kv_commit: the verifier's KV entries of the drafts, written to a scratch
  area, are committed to the cache only up to the accepted prefix (lesson,
  "KV 캐시 처리(KV cache dance)" and exercise 4).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "SequenceResult",
    "SampleResult",
    "tempered_log_normaliser",
    "tempered_probabilities",
    "first_argmax",
    "log_prob_of",
    "acceptance_ratio",
    "residual_weights",
    "bonus_weights",
    "inverse_cdf",
    "decision_margin",
    "cdf_margin",
    "verify_sequence",
    "verify_trials",
    "sample_row",
    "acceptance_rates",
    "kv_commit",
]


@dataclass
class SequenceResult:
    """Outputs of one verified sequence plus the oracle's decision margins."""

    n_accepted: int  # 0..N accepted draft tokens; -1 marks invalid input
    tokens: list  # N+1 entries: d_0..d_{j-1}, the drawn token, then -1s
    lse: list | None = None  # draft rows 0..N-1 then target rows 0..N; None at T = 0
    decision_margins: list = field(default_factory=list)  # one per accept test made
    sample_margin: float | None = None  # None at T = 0 (no draw)
    residual_mass: float | None = None  # S of the row that was drawn from


def tempered_log_normaliser(z_rows: np.ndarray, T: float) -> np.ndarray:
    """L = log sum_x exp(z_x / T) of each row, as max(x) + log sum exp(x - max(x))."""
    x = np.asarray(z_rows, dtype=np.float64) / T
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def tempered_probabilities(z_rows: np.ndarray, T: float) -> np.ndarray:
    """softmax(z / T) of each row: exp(z / T - L) with L the row's log-normaliser."""
    z = np.asarray(z_rows, dtype=np.float64)
    L = tempered_log_normaliser(z, T)
    return np.exp(z / T - L[..., None])


def first_argmax(row: np.ndarray) -> int:
    """Index of the largest entry; the lowest index wins a tie (numpy's argmax
    returns the first occurrence of the maximum)."""
    return int(np.argmax(np.asarray(row)))


def log_prob_of(z_row: np.ndarray, token: int, T: float, L: float) -> float:
    """log softmax(z / T)[token] given the row's log-normaliser L."""
    return float(z_row[token]) / T - L


def acceptance_ratio(log_q: float, log_p: float) -> float:
    """q(d) / p(d); infinite when the draft gave d zero probability, or when the
    ratio is beyond the fp64 range (then it exceeds every uniform)."""
    if log_p == -math.inf:
        return math.inf
    x = log_q - log_p
    return math.exp(x) if x < 709.0 else math.inf


def residual_weights(q: np.ndarray, p: np.ndarray) -> np.ndarray:
    """(q - p)_+ elementwise; the draw normalises it by its sum."""
    return np.maximum(0.0, q - p)


def bonus_weights(q: np.ndarray) -> np.ndarray:
    """The bonus token is drawn from the last verifier distribution itself."""
    return q


def cdf_margin(target: float, lower: float, upper: float) -> float:
    """Distance of ``target`` = u*S to the nearer edge of the chosen token's
    interval [lower, upper) = [C_{k-1}, C_k): how far the draw is from picking
    a neighbour."""
    return min(abs(target - lower), abs(upper - target))


def inverse_cdf(w: np.ndarray, u: float):
    """Draw a token from weights ``w`` with uniform ``u`` by an inverse CDF.

    Returns (token, margin, S): the smallest k with C_k > u*S, where
    C_k = sum_{x<=k} w_x in ascending token order and S = C_{V-1}; if rounding
    leaves none, the last k with w_k > 0. ``margin`` is cdf_margin of u*S in
    [C_{k-1}, C_k).
    """
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    S = float(C[-1])
    target = float(u) * S
    above = np.nonzero(C > target)[0]
    if above.size:
        k = int(above[0])
    else:
        k = int(np.nonzero(w > 0)[0][-1])
    lower = float(C[k - 1]) if k > 0 else 0.0
    return k, cdf_margin(target, lower, float(C[k])), S


def decision_margin(u: float, ratio: float) -> float:
    """Distance of an accept test u < ratio from its boundary: |u - ratio|
    (infinite when the ratio is, i.e. the draft gave the token zero mass)."""
    return abs(u - ratio)


def _valid_temperature(T: float) -> bool:
    return math.isfinite(T) and T >= 0.0


def _valid(T: float, tokens: np.ndarray, V: int) -> bool:
    if not _valid_temperature(T):
        return False
    return bool(np.all((tokens >= 0) & (tokens < V)))


def _invalid_result(N: int) -> SequenceResult:
    return SequenceResult(-1, [-1] * (N + 1))


def _emit(tokens: np.ndarray, j: int, drawn: int) -> list:
    N = len(tokens)
    return [int(t) for t in tokens[:j]] + [int(drawn)] + [-1] * (N - j)


def _verify_greedy(target_z: np.ndarray, tokens: np.ndarray) -> SequenceResult:
    N = len(tokens)
    g = [first_argmax(target_z[i]) for i in range(N + 1)]
    j = N
    for i in range(N):
        if int(tokens[i]) != g[i]:
            j = i
            break
    return SequenceResult(j, _emit(tokens, j, g[j]))


def _verify_sampled(draft_z, target_z, tokens, ua, us, T, Ld, Lt) -> SequenceResult:
    N = len(tokens)
    margins = []
    j = N
    for i in range(N):
        d = int(tokens[i])
        log_q = log_prob_of(target_z[i], d, T, Lt[i])
        log_p = log_prob_of(draft_z[i], d, T, Ld[i])
        ratio = acceptance_ratio(log_q, log_p)
        u = float(ua[i])
        margins.append(decision_margin(u, ratio))
        if not u < ratio:
            j = i
            break
    q_j = np.exp(np.asarray(target_z[j], dtype=np.float64) / T - Lt[j])
    if j < N:
        p_j = np.exp(np.asarray(draft_z[j], dtype=np.float64) / T - Ld[j])
        w = residual_weights(q_j, p_j)
        if not np.sum(w) > 0.0:
            w = q_j
    else:
        w = bonus_weights(q_j)
    k, smargin, S = inverse_cdf(w, float(us))
    lse = [float(v) for v in Ld] + [float(v) for v in Lt]
    return SequenceResult(j, _emit(tokens, j, k), lse, margins, smargin, S)


def verify_sequence(draft_z, target_z, tokens, accept_u, sample_u, T) -> SequenceResult:
    """Verify one sequence.

    draft_z [N, V] and target_z [N+1, V] are float64 logits (exactly widened
    from their storage type); tokens [N] ints; accept_u [N] and sample_u are
    the float32 uniforms widened to float64; T is the float32 temperature
    widened to float64.
    """
    draft_z = np.asarray(draft_z, dtype=np.float64)
    target_z = np.asarray(target_z, dtype=np.float64)
    tokens = np.asarray(tokens)
    N, V = target_z.shape[0] - 1, target_z.shape[1]
    T = float(T)
    if not _valid(T, tokens, V):
        return _invalid_result(N)
    if T == 0.0:
        return _verify_greedy(target_z, tokens)
    Ld = tempered_log_normaliser(draft_z, T)
    Lt = tempered_log_normaliser(target_z, T)
    return _verify_sampled(draft_z, target_z, tokens, accept_u, sample_u, T, Ld, Lt)


def verify_trials(draft_z, target_z, tokens, accept_u, sample_u, T) -> list:
    """Many sequences that share one set of logits (Monte-Carlo trials).

    draft_z [N, V] and target_z [N+1, V] are common to every trial; tokens
    [n, N], accept_u [n, N], sample_u [n] vary per trial. The per-row
    log-normalisers are computed once, since they depend on the logits only.
    """
    draft_z = np.asarray(draft_z, dtype=np.float64)
    target_z = np.asarray(target_z, dtype=np.float64)
    T = float(T)
    N, V = target_z.shape[0] - 1, target_z.shape[1]
    if T > 0.0 and math.isfinite(T):
        Ld = tempered_log_normaliser(draft_z, T)
        Lt = tempered_log_normaliser(target_z, T)
    out = []
    for n in range(tokens.shape[0]):
        if not _valid(T, tokens[n], V):
            out.append(_invalid_result(N))
        elif T == 0.0:
            out.append(_verify_greedy(target_z, tokens[n]))
        else:
            out.append(_verify_sampled(draft_z, target_z, tokens[n], accept_u[n], sample_u[n], T, Ld, Lt))
    return out


# ---------------------------------------------------------------------------
# Around the verification: the draft-side draw, acceptance telemetry and the
# KV-cache commit.


@dataclass
class SampleResult:
    """One drawn token plus the oracle's margin (None at T = 0 or when invalid)."""

    token: int  # -1 marks an invalid temperature
    margin: float | None = None


def sample_row(z_row, T: float, u: float) -> SampleResult:
    """Draw a token from softmax(z / T) with uniform u (the draft model's step).

    The lesson's draft loop draws each draft token from the draft model's
    tempered distribution; the draw here is the same inverse CDF as every
    other draw: the token is the smallest k with C_k > u * S over
    q = softmax(z / T) in ascending token order. T = 0 takes the first argmax
    (the low-temperature limit); a negative, NaN or infinite T gives -1.
    """
    z = np.asarray(z_row, dtype=np.float64)
    T = float(T)
    if not _valid_temperature(T):
        return SampleResult(-1)
    if T == 0.0:
        return SampleResult(first_argmax(z))
    q = tempered_probabilities(z, T)
    k, margin, _ = inverse_cdf(q, float(u))
    return SampleResult(k, margin)


def acceptance_rates(draft_z, target_z, tokens, T: float):
    """Per-position acceptance probability alpha_i and expected tokens per pass tau.

    alpha_i = sum_x min(p_i(x), q_i(x)): the probability that draft i is
    accepted given that position i is reached, when the draft token is drawn
    from p_i (the acceptance rule accepts x with probability min(1, q/p)).
    tau = sum_{k=0..N} prod_{i<k} alpha_i is the expected number of tokens one
    verifier pass emits: position k is reached with probability
    prod_{i<k} alpha_i and every reached position emits one token (the last
    one the correction or the bonus). With alpha constant this is
    (1 - alpha^(N+1)) / (1 - alpha), the lesson's closed form.
    At T = 0 both distributions are point masses (the draft's greedy pick d_i
    and the verifier's first argmax g_i), so alpha_i = 1 if d_i = g_i else 0.
    Returns (alpha [N] list, tau); NaNs when the sequence is invalid.
    """
    draft_z = np.asarray(draft_z, dtype=np.float64)
    target_z = np.asarray(target_z, dtype=np.float64)
    tokens = np.asarray(tokens)
    N, V = target_z.shape[0] - 1, target_z.shape[1]
    T = float(T)
    if not _valid(T, tokens, V):
        return [math.nan] * N, math.nan
    if T == 0.0:
        alpha = [1.0 if int(tokens[i]) == first_argmax(target_z[i]) else 0.0 for i in range(N)]
    else:
        p = tempered_probabilities(draft_z, T)
        q = tempered_probabilities(target_z[:N], T)
        alpha = [float(np.sum(np.minimum(p[i], q[i]))) for i in range(N)]
    tau = 0.0
    reach = 1.0
    for k in range(N + 1):
        tau += reach
        if k < N:
            reach *= alpha[k]
    return alpha, tau


def kv_commit(cache, cache_len, scratch, n_accepted):
    """Commit the accepted drafts' KV entries from a scratch area into the cache.

    The verifier's pass over N drafts writes one KV entry per draft into a
    scratch area; once n = n_accepted of them are accepted, entries 0..n-1 are
    appended to the sequence's cache at its current length and the length
    grows by n, so the next pass reads the prefix plus the accepted drafts and
    nothing of the rejected ones (lesson, "KV 캐시 처리(KV cache dance)";
    exercise 4 checks exactly this).

    cache [P, B, L, E] and scratch [P, B, N, E] are byte arrays (P planes, e.g.
    keys and values of every layer; E bytes per entry); cache_len and
    n_accepted [B]. A sequence whose n_accepted is outside [0, N] (an invalid
    verification) or whose entries would not fit (len + n > L, or len < 0) is
    left as it is and reports length -1. Returns (new cache, new lengths);
    the inputs are not modified.
    """
    out = np.array(cache, copy=True)
    scratch = np.asarray(scratch)
    P, B, L, E = out.shape
    N = scratch.shape[2]
    new_len = np.empty(B, dtype=np.int64)
    for b in range(B):
        n = int(n_accepted[b])
        start = int(cache_len[b])
        if n < 0 or n > N or start < 0 or start + n > L:
            new_len[b] = -1
            continue
        for p in range(P):
            for t in range(n):
                out[p, b, start + t, :] = scratch[p, b, t, :]
        new_len[b] = start + n
    return out, new_len
