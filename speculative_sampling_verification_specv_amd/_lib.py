"""ctypes binding of libspecv: argument marshalling only.

The functions carry the C entry points' names and take torch tensors (for
device memory) and a torch stream. Every step of the verification runs in the
HIP library; nothing here computes. The contract of each call (layouts,
ownership, error codes) is documented in include/specv.h.
"""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

SPECV_F32 = 0
SPECV_BF16 = 1
SPECV_OK = 0
SPECV_EINVAL = -1
SPECV_ENOMEM = -2
SPECV_EHIP = -3
SPECV_EALIGN = -4
SPECV_ESTATE = -5
SPECV_ERANGE = -6
SPECV_MAX_DRAFT = 64
SPECV_MAX_VOCAB = 1 << 18

# Entry points declared in include/specv.h, with their ctypes signatures.
_SIGNATURES = {
    "specv_create": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int]),
    "specv_verify": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 9),
    "specv_verify_lazy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 9),
    "specv_verify_static": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
                            + [ctypes.c_void_p] * 9),
    "specv_row_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "specv_sample": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 5),
    "specv_acceptance_rates": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 7),
    "specv_kv_commit": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "specv_destroy": (None, [ctypes.c_void_p]),
    "specv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "specv_set_timing": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "specv_set_wait_limit": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "specv_last_timings": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int)]),
    "specv_stage_name": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class SpecvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {specv_strerror(code)} ({code})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecv.so once. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -m speculative_sampling_verification_specv_amd.build)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(code: int, what: str) -> None:
    if code != SPECV_OK:
        raise SpecvError(code, what)


def _ptr(t) -> int:
    return int(t.data_ptr())


def _stream_ptr(stream, device) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def specv_strerror(code: int) -> str:
    return load_library().specv_strerror(int(code)).decode()


def specv_create(max_batch: int, max_draft: int, vocab: int, dtype: int, device: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(load_library().specv_create(ctypes.byref(h), max_batch, max_draft, vocab, dtype, device),
           "specv_create")
    return int(h.value)


def specv_destroy(handle: int) -> None:
    load_library().specv_destroy(handle)


def specv_verify(handle: int, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms,
                 temperature, out_tokens, out_n_accepted, stream=None) -> None:
    """Enqueue one verification; batch and n_draft come from draft_tokens' shape."""
    B, N = draft_tokens.shape
    _check(load_library().specv_verify(
        handle, int(B), int(N), _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens),
        _ptr(accept_uniforms), _ptr(sample_uniforms), _ptr(temperature), _ptr(out_tokens),
        _ptr(out_n_accepted), _stream_ptr(stream, draft_tokens.device)), "specv_verify")


def specv_verify_lazy(handle: int, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms,
                      temperature, out_tokens, out_n_accepted, stream=None) -> None:
    """Enqueue one lazy verification (rows read up to each sequence's first rejection)."""
    B, N = draft_tokens.shape
    _check(load_library().specv_verify_lazy(
        handle, int(B), int(N), _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens),
        _ptr(accept_uniforms), _ptr(sample_uniforms), _ptr(temperature), _ptr(out_tokens),
        _ptr(out_n_accepted), _stream_ptr(stream, draft_tokens.device)), "specv_verify_lazy")


def specv_verify_static(draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms, temperature,
                        out_tokens, out_n_accepted, stream=None) -> None:
    """Enqueue one verification through the allocation-free entry point (no handle).

    batch and n_draft come from draft_tokens' shape, the vocabulary from the
    logits' last dimension and the dtype from theirs; the tensors' layouts are
    those of specv_verify (the caller checks them)."""
    import torch

    B, N = draft_tokens.shape
    V = int(target_logits.shape[-1])
    dtype = SPECV_F32 if target_logits.dtype == torch.float32 else SPECV_BF16
    _check(load_library().specv_verify_static(
        int(B), int(N), V, dtype, _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens),
        _ptr(accept_uniforms), _ptr(sample_uniforms), _ptr(temperature), _ptr(out_tokens),
        _ptr(out_n_accepted), _stream_ptr(stream, draft_tokens.device)), "specv_verify_static")


def specv_sample(handle: int, logits, temperature, uniforms, out_tokens, stream=None) -> None:
    """Enqueue one draw per row of logits [n_rows, V]."""
    n = int(logits.shape[0])
    _check(load_library().specv_sample(handle, n, _ptr(logits), _ptr(temperature), _ptr(uniforms), _ptr(out_tokens),
                                       _stream_ptr(stream, logits.device)), "specv_sample")


def specv_kv_commit(cache, cache_len, scratch, n_accepted, out_cache_len, stream=None) -> None:
    """Enqueue the KV-cache commit of the accepted drafts.

    cache [P, B, L, ...] and scratch [P, B, N, ...] are device tensors of one
    dtype whose trailing dimensions (one entry) match; each (plane, sequence)
    slice must be contiguous. cache_len, n_accepted, out_cache_len: int32 [B].
    """
    if cache.dtype != scratch.dtype or tuple(cache.shape[3:]) != tuple(scratch.shape[3:]):
        raise ValueError("cache and scratch entries differ in dtype or shape")
    if tuple(cache.shape[:2]) != tuple(scratch.shape[:2]):
        raise ValueError("cache and scratch differ in planes or batch")
    P, B, L = (int(x) for x in cache.shape[:3])
    N = int(scratch.shape[2])
    entry_elems = 1
    for x in cache.shape[3:]:
        entry_elems *= int(x)
    es = cache.element_size()
    for t, name in ((cache, "cache"), (scratch, "scratch")):
        inner = 1
        for d in range(t.dim() - 1, 1, -1):
            if t.stride(d) != inner:
                raise ValueError(f"{name}: each (plane, sequence) slice must be contiguous")
            inner *= int(t.shape[d])
    _check(load_library().specv_kv_commit(
        P, B, N, L, entry_elems * es, _ptr(cache), cache.stride(0) * es, cache.stride(1) * es,
        _ptr(scratch), scratch.stride(0) * es, scratch.stride(1) * es, _ptr(n_accepted), _ptr(cache_len),
        _ptr(out_cache_len), _stream_ptr(stream, cache.device)), "specv_kv_commit")


def specv_acceptance_rates(handle: int, draft_logits, target_logits, draft_tokens, temperature, out_alpha, out_tau,
                           stream=None) -> None:
    B, N = draft_tokens.shape
    _check(load_library().specv_acceptance_rates(
        handle, int(B), int(N), _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens), _ptr(temperature),
        _ptr(out_alpha), _ptr(out_tau), _stream_ptr(stream, draft_tokens.device)), "specv_acceptance_rates")


def specv_row_stats(handle: int, out_lse, out_argmax, stream=None) -> None:
    _check(load_library().specv_row_stats(handle, _ptr(out_lse), _ptr(out_argmax),
                                          _stream_ptr(stream, out_lse.device)), "specv_row_stats")


def specv_set_wait_limit(handle: int, microseconds: int) -> None:
    _check(load_library().specv_set_wait_limit(handle, int(microseconds)), "specv_set_wait_limit")


def specv_set_timing(handle: int, enable: bool) -> None:
    _check(load_library().specv_set_timing(handle, 1 if enable else 0), "specv_set_timing")


def specv_last_timings(handle: int) -> dict:
    """{stage name: milliseconds} of the most recent timed verify (waits for it)."""
    ms = (ctypes.c_float * 16)()
    n = ctypes.c_int()
    _check(load_library().specv_last_timings(handle, ms, 16, ctypes.byref(n)), "specv_last_timings")
    return {specv_stage_name(i): float(ms[i]) for i in range(n.value)}


def specv_stage_name(stage: int) -> str | None:
    name = load_library().specv_stage_name(int(stage))
    return None if name is None else name.decode()


class Verifier:
    """One library handle plus shape/dtype checks of the torch tensors handed to it."""

    def __init__(self, max_batch: int, max_draft: int, vocab: int, dtype: str = "bf16", device: int = 0):
        import torch

        self.max_batch, self.max_draft, self.vocab = int(max_batch), int(max_draft), int(vocab)
        self.dtype = dtype
        self.torch_dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
        self.device = torch.device("cuda", device)
        self.handle = specv_create(self.max_batch, self.max_draft, self.vocab,
                                   SPECV_F32 if dtype == "f32" else SPECV_BF16, device)
        self._last = None

    def close(self) -> None:
        if getattr(self, "handle", None):
            specv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _expect(self, t, name, shape, dtype):
        if t.device != self.device:
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def verify(self, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms, temperature,
               out_tokens=None, out_n_accepted=None, stream=None):
        """Verify a batch; returns (out_tokens [B, N+1] int32, out_n_accepted [B] int32)."""
        import torch

        B, N = draft_tokens.shape
        V = self.vocab
        self._expect(draft_logits, "draft_logits", (B, N, V), self.torch_dtype)
        self._expect(target_logits, "target_logits", (B, N + 1, V), self.torch_dtype)
        self._expect(draft_tokens, "draft_tokens", (B, N), torch.int32)
        self._expect(accept_uniforms, "accept_uniforms", (B, N), torch.float32)
        self._expect(sample_uniforms, "sample_uniforms", (B,), torch.float32)
        self._expect(temperature, "temperature", (B,), torch.float32)
        if out_tokens is None:
            out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=self.device)
        if out_n_accepted is None:
            out_n_accepted = torch.empty((B,), dtype=torch.int32, device=self.device)
        self._expect(out_tokens, "out_tokens", (B, N + 1), torch.int32)
        self._expect(out_n_accepted, "out_n_accepted", (B,), torch.int32)
        specv_verify(self.handle, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms,
                     temperature, out_tokens, out_n_accepted, stream)
        self._last = (B, N)
        return out_tokens, out_n_accepted

    def verify_lazy(self, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms, temperature,
                    out_tokens=None, out_n_accepted=None, stream=None):
        """verify() that reads each sequence's rows only up to its first rejection (same results)."""
        import torch

        B, N = draft_tokens.shape
        V = self.vocab
        self._expect(draft_logits, "draft_logits", (B, N, V), self.torch_dtype)
        self._expect(target_logits, "target_logits", (B, N + 1, V), self.torch_dtype)
        self._expect(draft_tokens, "draft_tokens", (B, N), torch.int32)
        self._expect(accept_uniforms, "accept_uniforms", (B, N), torch.float32)
        self._expect(sample_uniforms, "sample_uniforms", (B,), torch.float32)
        self._expect(temperature, "temperature", (B,), torch.float32)
        if out_tokens is None:
            out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=self.device)
        if out_n_accepted is None:
            out_n_accepted = torch.empty((B,), dtype=torch.int32, device=self.device)
        self._expect(out_tokens, "out_tokens", (B, N + 1), torch.int32)
        self._expect(out_n_accepted, "out_n_accepted", (B,), torch.int32)
        specv_verify_lazy(self.handle, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms,
                          temperature, out_tokens, out_n_accepted, stream)
        self._last = (B, N)
        return out_tokens, out_n_accepted

    def bind(self, draft_logits, target_logits, draft_tokens, accept_uniforms, sample_uniforms, temperature,
             out_tokens, out_n_accepted, stream=None, lazy: bool = False):
        """Check one call's arguments once; return a function that enqueues exactly that call.

        The returned function re-issues specv_verify with the same buffers and
        stream and no per-call Python checks, for loops that refill the same
        tensors in place (the caller keeps them alive). It raises SpecvError on
        a nonzero status.
        """
        import torch

        B, N = draft_tokens.shape
        V = self.vocab
        self._expect(draft_logits, "draft_logits", (B, N, V), self.torch_dtype)
        self._expect(target_logits, "target_logits", (B, N + 1, V), self.torch_dtype)
        self._expect(draft_tokens, "draft_tokens", (B, N), torch.int32)
        self._expect(accept_uniforms, "accept_uniforms", (B, N), torch.float32)
        self._expect(sample_uniforms, "sample_uniforms", (B,), torch.float32)
        self._expect(temperature, "temperature", (B,), torch.float32)
        self._expect(out_tokens, "out_tokens", (B, N + 1), torch.int32)
        self._expect(out_n_accepted, "out_n_accepted", (B,), torch.int32)
        fn = load_library().specv_verify_lazy if lazy else load_library().specv_verify
        args = (self.handle, int(B), int(N), _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens),
                _ptr(accept_uniforms), _ptr(sample_uniforms), _ptr(temperature), _ptr(out_tokens),
                _ptr(out_n_accepted), _stream_ptr(stream, draft_tokens.device))
        self._last = (int(B), int(N))

        def call() -> None:
            rc = fn(*args)
            if rc != SPECV_OK:
                raise SpecvError(rc, "specv_verify")

        return call

    def sample(self, logits, temperature, uniforms, out_tokens=None, stream=None):
        """Draw one token per row of logits [n_rows, V]; returns out_tokens [n_rows] int32."""
        import torch

        n = int(logits.shape[0])
        self._expect(logits, "logits", (n, self.vocab), self.torch_dtype)
        self._expect(temperature, "temperature", (n,), torch.float32)
        self._expect(uniforms, "uniforms", (n,), torch.float32)
        if out_tokens is None:
            out_tokens = torch.empty((n,), dtype=torch.int32, device=self.device)
        self._expect(out_tokens, "out_tokens", (n,), torch.int32)
        specv_sample(self.handle, logits, temperature, uniforms, out_tokens, stream)
        self._last = (n, 0)
        return out_tokens

    def acceptance_rates(self, draft_logits, target_logits, draft_tokens, temperature, stream=None):
        """(alpha [B, N], tau [B]) float32 of the last verify (same tensors, unchanged)."""
        import torch

        B, N = draft_tokens.shape
        alpha = torch.empty((B, N), dtype=torch.float32, device=self.device)
        tau = torch.empty((B,), dtype=torch.float32, device=self.device)
        specv_acceptance_rates(self.handle, draft_logits, target_logits, draft_tokens, temperature, alpha, tau, stream)
        return alpha, tau

    def set_timing(self, enable: bool) -> None:
        specv_set_timing(self.handle, enable)

    def set_wait_limit(self, microseconds: int) -> None:
        specv_set_wait_limit(self.handle, microseconds)

    def last_timings(self) -> dict:
        return specv_last_timings(self.handle)

    def row_stats(self, stream=None):
        """(lse [B, 2N+1] float32, argmax [B, 2N+1] int32) of the last verify."""
        import torch

        if self._last is None:
            raise SpecvError(SPECV_ESTATE, "row_stats")
        B, N = self._last
        lse = torch.empty((B, 2 * N + 1), dtype=torch.float32, device=self.device)
        amax = torch.empty((B, 2 * N + 1), dtype=torch.int32, device=self.device)
        specv_row_stats(self.handle, lse, amax, stream)
        return lse, amax
