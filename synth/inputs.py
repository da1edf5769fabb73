"""Seeded synthetic inputs for batched speculative-sampling verification.

No trained draft or verifier model is available, so their logits are
synthesised the way the speculative-decoding lesson page ("추측 디코딩 — 초안
작성, 검증, 반복", section "직접 만들기") fakes its models: a fixed verifier
distribution and a draft that is a perturbation of it.

* Verifier (target) logits at every position: ``scale * N(0, 1)`` per token,
  minus ``s * ln(rank)`` where ``rank`` is a fresh random permutation of
  ``1..V`` (a Zipf log-prior, as real LM heads are heavy-headed). Positions
  0..N are independent rows.
* Draft logits at position i < N: the target logits of position i plus
  ``sigma_b * N(0, 1)`` noise; ``sigma_b`` is drawn per sequence and sets how
  well the draft matches the target.
* Both are rounded to the storage type (float32, or bfloat16 with
  round-to-nearest-even). bfloat16 data is carried as raw ``uint16`` bits.
* Draft tokens are drawn from the tempered draft distribution by the
  Gumbel-max trick (``argmax_x z_x / T + G_x`` with ``G = -log(-log U)``); at
  temperature 0 they are the first argmax of the draft row.
* Uniforms are ``k * 2**-24`` with ``k`` uniform in ``[0, 2**24)``, so they are
  exact in float32 and lie in [0, 1).

This module holds none of the verification arithmetic (no softmax normaliser,
no acceptance test, no residual, no inverse CDF). Both the HIP library and the
oracle consume its arrays; it imports neither.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload",
    "Batch",
    "WORKLOADS",
    "workload",
    "make_batch",
    "make_trials",
    "resample",
    "SampleRows",
    "make_sample_rows",
    "widen",
    "to_bf16_bits",
    "gumbel_max_tokens",
    "grid_uniforms",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic verification workload (shape plus generator recipe)."""

    name: str
    index: int  # first element of every seed sequence drawn for this workload
    batch: int
    n_draft: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    scale: float  # std of the Gaussian part of the target logits
    zipf_s: float  # exponent of the Zipf log-prior; 0 disables it
    sigma: tuple  # (lo, hi): per-sequence draft noise std ~ U(lo, hi)
    temperature: tuple  # (T for even sequences, T for odd sequences)

    def with_sizes(self, batch: int | None = None, vocab: int | None = None,
                   n_draft: int | None = None) -> "Workload":
        """The same generator at other sizes (small parity cases)."""
        return replace(
            self,
            batch=self.batch if batch is None else int(batch),
            vocab=self.vocab if vocab is None else int(vocab),
            n_draft=self.n_draft if n_draft is None else int(n_draft),
        )

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w
    for w in (
        # A single 16-token sequence; also the base of the 10^5-trial Monte Carlo.
        Workload("tiny_b1_n4_v16_f32", 1, 1, 4, 16, "f32", 1.0, 0.0, (0.5, 0.5), (1.0, 1.0)),
        # One sequence over a 32000-token vocabulary (acceptance rate about 0.7).
        Workload("b1_n5_v32000_f32", 2, 1, 5, 32000, "f32", 2.5, 1.1, (0.7, 0.7), (1.0, 1.0)),
        # 64 sequences, 128256-token vocabulary, bfloat16 logits, T = 0.7.
        Workload("b64_n5_v128256_bf16", 3, 64, 5, 128256, "bf16", 3.0, 1.2, (0.2, 1.5), (0.7, 0.7)),
        # 256 sequences, 151936-token vocabulary, greedy (even b) and T = 1 (odd b).
        Workload("b256_n7_v151936_bf16_mixed", 4, 256, 7, 151936, "bf16", 2.5, 1.1, (0.1, 1.0), (0.0, 1.0)),
        # 32 sequences drafting 16 tokens each with a poor draft (early rejections).
        Workload("b32_n16_v128256_f32", 5, 32, 16, 128256, "f32", 2.5, 1.1, (2.0, 2.0), (1.0, 1.0)),
    )
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass
class Batch:
    """Host arrays of one verification call, in the layouts the library takes.

    draft_logits   [B, N, V]    float32, or uint16 bfloat16 bits
    target_logits  [B, N+1, V]  same storage type
    draft_tokens   [B, N]       int32
    accept_uniforms[B, N]       float32 in [0, 1)
    sample_uniforms[B]          float32 in [0, 1)
    temperature    [B]          float32, >= 0 (0 = greedy)
    """

    dtype: str
    draft_logits: np.ndarray
    target_logits: np.ndarray
    draft_tokens: np.ndarray
    accept_uniforms: np.ndarray
    sample_uniforms: np.ndarray
    temperature: np.ndarray

    @property
    def batch(self) -> int:
        return int(self.draft_tokens.shape[0])

    @property
    def n_draft(self) -> int:
        return int(self.draft_tokens.shape[1])

    @property
    def vocab(self) -> int:
        return int(self.target_logits.shape[-1])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + rounding) >> np.uint32(16)).astype(np.uint16)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored logits (float32 or bfloat16 bits) to float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _quantise(x32: np.ndarray, dtype: str) -> np.ndarray:
    return x32.astype(np.float32) if dtype == "f32" else to_bf16_bits(x32)


def grid_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms on the k * 2^-24 grid, exact in float32, in [0, 1)."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_max_tokens(z64: np.ndarray, temperature: float, rng: np.random.Generator) -> np.ndarray:
    """Draw one token per row of ``z64`` from softmax(z / T) by the Gumbel-max trick.

    ``argmax_x (z_x / T + G_x)`` with i.i.d. standard Gumbel ``G_x`` is an exact
    draw from the tempered softmax; no normaliser is ever formed. At T == 0 the
    first argmax of the row is returned.
    """
    z64 = np.atleast_2d(np.asarray(z64, dtype=np.float64))
    if temperature == 0.0:
        return np.argmax(z64, axis=-1).astype(np.int32)
    u = rng.random(z64.shape)
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))  # u == 0 gives -inf: that token is never picked
    return np.argmax(z64 / float(temperature) + g, axis=-1).astype(np.int32)


def _sequence_temperature(wl: Workload, b: int) -> np.float32:
    return np.float32(wl.temperature[b % 2])


def make_batch(wl: Workload, seed: int) -> Batch:
    """All arrays of one call of workload ``wl``, reproducible from ``seed``."""
    B, N, V = wl.batch, wl.n_draft, wl.vocab
    rng = np.random.default_rng(np.random.SeedSequence([wl.index, int(seed)]))
    store = np.float32 if wl.dtype == "f32" else np.uint16
    draft = np.empty((B, N, V), dtype=store)
    target = np.empty((B, N + 1, V), dtype=store)
    tokens = np.empty((B, N), dtype=np.int32)
    temps = np.empty((B,), dtype=np.float32)
    log_rank = np.log(np.arange(1, V + 1, dtype=np.float64)).astype(np.float32)
    for b in range(B):
        lo, hi = wl.sigma
        sigma = np.float32(lo if lo == hi else rng.uniform(lo, hi))
        temps[b] = _sequence_temperature(wl, b)
        t32 = rng.standard_normal((N + 1, V), dtype=np.float32) * np.float32(wl.scale)
        if wl.zipf_s != 0.0:
            for i in range(N + 1):
                t32[i] -= np.float32(wl.zipf_s) * log_rank[rng.permutation(V)]
        d32 = t32[:N] + sigma * rng.standard_normal((N, V), dtype=np.float32)
        target[b] = _quantise(t32, wl.dtype)
        draft[b] = _quantise(d32, wl.dtype)
        tokens[b] = gumbel_max_tokens(widen(draft[b], wl.dtype), float(temps[b]), rng)
    accept_u = grid_uniforms(rng, (B, N))
    sample_u = grid_uniforms(rng, (B,))
    return Batch(wl.dtype, draft, target, tokens, accept_u, sample_u, temps)


def make_trials(wl: Workload, seed: int, n_trials: int) -> Batch:
    """``n_trials`` sequences that share one sequence's logits.

    The logits of sequence 0 of ``make_batch(wl, seed)`` are repeated for every
    trial; each trial draws its own draft tokens (from that fixed draft
    distribution) and its own uniforms. This is the Monte-Carlo setting in
    which the emitted tokens must follow the verifier distribution.
    """
    base = make_batch(wl.with_sizes(batch=1), seed)
    rng = np.random.default_rng(np.random.SeedSequence([wl.index, int(seed), 1]))
    T = float(base.temperature[0])
    d64 = widen(base.draft_logits[0], wl.dtype)
    N = wl.n_draft
    tokens = np.empty((n_trials, N), dtype=np.int32)
    for i in range(N):
        rows = np.broadcast_to(d64[i], (n_trials, d64.shape[-1]))
        tokens[:, i] = gumbel_max_tokens(rows, T, rng)
    return Batch(
        wl.dtype,
        np.broadcast_to(base.draft_logits, (n_trials,) + base.draft_logits.shape[1:]),
        np.broadcast_to(base.target_logits, (n_trials,) + base.target_logits.shape[1:]),
        tokens,
        grid_uniforms(rng, (n_trials, N)),
        grid_uniforms(rng, (n_trials,)),
        np.full((n_trials,), base.temperature[0], dtype=np.float32),
    )


def resample(batch: Batch, wl: Workload, seed: int, variant: int) -> Batch:
    """The same logits with fresh draft tokens and uniforms.

    Variant 0 is ``batch`` itself; variant v > 0 draws every sequence's draft
    tokens again from its tempered draft distribution (Gumbel-max) and new
    accept and sample uniforms, from a seed of its own. Many verification
    cases then share one set of logits (one upload, one set of row
    normalisers) while their decisions and draws differ.
    """
    if variant == 0:
        return batch
    rng = np.random.default_rng(np.random.SeedSequence([wl.index, int(seed), 1000 + int(variant)]))
    B, N = batch.batch, batch.n_draft
    tokens = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        tokens[b] = gumbel_max_tokens(widen(batch.draft_logits[b], batch.dtype), float(batch.temperature[b]), rng)
    return Batch(batch.dtype, batch.draft_logits, batch.target_logits, tokens, grid_uniforms(rng, (B, N)),
                 grid_uniforms(rng, (B,)), batch.temperature)


@dataclass
class SampleRows:
    """Host arrays of one draft-side draw: rows of logits, a temperature and a uniform per row."""

    dtype: str
    logits: np.ndarray  # [n, V] float32 or uint16 bfloat16 bits
    temperature: np.ndarray  # [n] float32
    uniforms: np.ndarray  # [n] float32 in [0, 1)


def make_sample_rows(wl: Workload, seed: int, n_rows: int) -> SampleRows:
    """``n_rows`` draft-model rows of workload ``wl`` (its draft logits, position
    after position, sequence after sequence) with the sequences' temperatures
    and fresh uniforms."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.index, int(seed), 2]))
    B = -(-n_rows // wl.n_draft)
    b = make_batch(wl.with_sizes(batch=B), seed)
    logits = np.ascontiguousarray(b.draft_logits.reshape(B * wl.n_draft, wl.vocab)[:n_rows])
    temps = np.repeat(b.temperature, wl.n_draft)[:n_rows].astype(np.float32)
    return SampleRows(wl.dtype, logits, temps, grid_uniforms(rng, (n_rows,)))
