"""GPU acceptance telemetry (specv_acceptance_rates) against oracle.acceptance_rates.

alpha_i and tau per sequence after a verification, to 1e-5 absolute (the
library forms p and q from fp64 arguments and exponentiates them in fp32);
greedy sequences exactly (0 or 1), invalid ones NaN.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import require_gpu, to_device
from speculative_sampling_verification_specv_amd import SpecvError, Verifier, _lib

pytestmark = pytest.mark.gpu

ATOL = 1e-5


def _rates(batch):
    dev = require_gpu()
    args = to_device(batch, dev)
    with Verifier(batch.batch, batch.n_draft, batch.vocab, batch.dtype) as v:
        v.verify(**args)
        alpha, tau = v.acceptance_rates(args["draft_logits"], args["target_logits"], args["draft_tokens"],
                                        args["temperature"])
        torch.cuda.synchronize()
    return alpha.cpu().numpy(), tau.cpu().numpy()


def _check(batch, alpha, tau, label):
    N = batch.n_draft
    for s in range(batch.batch):
        T = float(batch.temperature[s])
        want_a, want_t = oracle.acceptance_rates(synth.widen(batch.draft_logits[s], batch.dtype),
                                                 synth.widen(batch.target_logits[s], batch.dtype),
                                                 batch.draft_tokens[s], T)
        if np.isnan(want_t) or (0.0 < T < 2.0 ** -60):
            assert np.all(np.isnan(alpha[s])) and np.isnan(tau[s]), (label, s)
            continue
        if T == 0.0:
            assert alpha[s].tolist() == want_a and tau[s] == np.float32(want_t), (label, s)
            continue
        assert np.max(np.abs(alpha[s] - np.asarray(want_a))) <= ATOL, (label, s, alpha[s], want_a)
        assert abs(tau[s] - want_t) <= ATOL * (N + 1), (label, s, tau[s], want_t)


@pytest.mark.parametrize("name,batch,vocab", [
    ("b64_n5_v128256_bf16", 16, 3 * 32768 + 517),
    ("b256_n7_v151936_bf16_mixed", 12, 2 * 32768 + 4099),
    ("b32_n16_v128256_f32", 6, 3 * 16384 + 37),
    ("b1_n5_v32000_f32", 1, 32000),
    ("tiny_b1_n4_v16_f32", 1, 16),
])
def test_rates_match_oracle(name, batch, vocab):
    wl = synth.workload(name).with_sizes(batch=batch, vocab=vocab)
    b = synth.make_batch(wl, seed=5)
    alpha, tau = _rates(b)
    _check(b, alpha, tau, name)


def test_rates_full_size():
    wl = synth.workload("b64_n5_v128256_bf16")
    b = synth.make_batch(wl, seed=7)
    alpha, tau = _rates(b)
    _check(b, alpha, tau, "full")
    print(f"[rates] B=64: mean alpha {np.nanmean(alpha):.4f}, mean tau {np.nanmean(tau):.3f}", flush=True)


def test_rates_closed_form():
    """Every position with the same (p, q): alpha constant, tau = (1 - a^(N+1)) / (1 - a)."""
    N, V = 5, 2048
    rng = np.random.default_rng(4)
    zt = rng.normal(size=V).astype(np.float32) * 2
    zd = (zt + rng.normal(size=V).astype(np.float32) * 0.8).astype(np.float32)
    b = synth.Batch("f32", np.tile(zd, (2, N, 1)), np.tile(zt, (2, N + 1, 1)),
                    np.zeros((2, N), np.int32), np.zeros((2, N), np.float32), np.zeros(2, np.float32),
                    np.array([1.0, 0.6], np.float32))
    alpha, tau = _rates(b)
    for s in range(2):
        a = float(alpha[s, 0])
        assert np.allclose(alpha[s], a, atol=1e-7)
        assert abs(tau[s] - (1 - a ** (N + 1)) / (1 - a)) < 1e-5
    _check(b, alpha, tau, "closed form")


def test_rates_invalid_and_state():
    dev = require_gpu()
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(batch=5, vocab=700, n_draft=3)
    b = synth.make_batch(wl, seed=2)
    b.temperature[:] = np.array([1.0, np.nan, 0.0, 1e-30, 0.5], dtype=np.float32)
    b.draft_tokens[4, 1] = 700
    alpha, tau = _rates(b)
    _check(b, alpha, tau, "invalid")
    assert np.all(np.isnan(alpha[[1, 3, 4]])) and np.all(np.isnan(tau[[1, 3, 4]]))
    # A handle whose last call had another shape refuses.
    args = to_device(b, dev)
    with Verifier(5, 4, 700, "f32") as v:
        with pytest.raises(SpecvError) as e:
            v.acceptance_rates(args["draft_logits"], args["target_logits"], args["draft_tokens"], args["temperature"])
        assert e.value.code == _lib.SPECV_ESTATE
