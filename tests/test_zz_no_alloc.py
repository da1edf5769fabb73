"""The allocation-free entry point against the handle-based one.

specv_verify_static (no handle, a static device workspace) must give exactly
what specv_verify gives on the same inputs (both run the same kernels), on two
calls in a row, the second smaller than the first, and both must match the
oracle by the parity rules.
"""

import numpy as np
import pytest
import torch

import synth
from parity import GpuResult, compare, require_gpu, run_gpu, run_oracle, to_device
from speculative_sampling_verification_specv_amd import SpecvError, Verifier, _lib

pytestmark = pytest.mark.gpu


def _static_call(batch, dev):
    args = to_device(batch, dev)
    B, N = batch.batch, batch.n_draft
    out_t = torch.full((B, N + 1), -7, dtype=torch.int32, device=dev)
    out_n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    _lib.specv_verify_static(args["draft_logits"], args["target_logits"], args["draft_tokens"],
                             args["accept_uniforms"], args["sample_uniforms"], args["temperature"], out_t, out_n)
    torch.cuda.synchronize()
    return out_t.cpu().numpy(), out_n.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (("b64_n5_v128256_bf16", 24, 40000, 3), ("b64_n5_v128256_bf16", 7, 40000, 4)),
    (("b256_n7_v151936_bf16_mixed", 32, 151936, 5), ("b1_n5_v32000_f32", 3, 9001, 6)),
    (("b32_n16_v128256_f32", 16, 70001, 7), ("b256_n7_v151936_bf16_mixed", 5, 3000, 8)),
])
def test_static_entry_matches_handle(first, second):
    dev = require_gpu()
    for name, B, V, seed in (first, second):
        wl = synth.workload(name).with_sizes(batch=B, vocab=V)
        b = synth.make_batch(wl, seed)
        toks, nacc = _static_call(b, dev)
        with Verifier(B, wl.n_draft, V, wl.dtype) as v:
            ref = run_gpu(b, v)
        assert np.array_equal(nacc, ref.n_accepted), (name, B, V)
        assert np.array_equal(toks, ref.tokens), (name, B, V)
        compare(b, GpuResult(toks, nacc, None, None), run_oracle(b)).check(f"static {name} B={B} V={V}")


def test_static_entry_limits():
    dev = require_gpu()
    wl = synth.workload("b1_n5_v32000_f32").with_sizes(batch=2, vocab=64)
    b = synth.make_batch(wl, 1)
    args = to_device(b, dev)
    out_t = torch.empty((257, 6), dtype=torch.int32, device=dev)
    out_n = torch.empty((257,), dtype=torch.int32, device=dev)
    big = torch.zeros((257, 5), dtype=torch.int32, device=dev)
    with pytest.raises(SpecvError) as e:
        _lib.specv_verify_static(args["draft_logits"], args["target_logits"], big, args["accept_uniforms"],
                                 args["sample_uniforms"], args["temperature"], out_t, out_n)
    assert e.value.code == _lib.SPECV_ERANGE
