"""MI355X-native lookahead decoding: thin Python binding of liblaamd.so.

The binding only marshals arguments: every step of the decoding path runs in
the library's HIP kernels.  PyTorch provides device memory (weights,
workspace) and the stream.  Importing works without a GPU; creating a
decoder needs the built library and a gfx950 device, and fails loudly
otherwise (there is no CPU fallback).

Method: "Break the Sequential Dependency of LLM Inference Using Lookahead
Decoding" (Fu et al. 2024), summary page (Summary; Key points, "Tuning
knobs").  The C ABI is documented in include/la.h.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB as _LIB_PATH, build  # noqa: F401

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_STATE = 0, -1, -2
LA_ERR_OUT_OF_CAPACITY, LA_ERR_HIP, LA_ERR_UNSUPPORTED = -3, -4, -5
# device scratch of la_attention_noalloc (include/la.h)
LA_ATTENTION_NOALLOC_SCRATCH_BYTES = 16 << 20
LA_F32, LA_BF16 = 0, 1

EXPORTS = [
    "la_workspace_bytes", "la_create", "la_prefill", "la_step", "la_step_submit",
    "la_step_collect", "la_destroy",
    "la_status_string", "la_last_error", "la_step_rows", "la_debug_logits",
    "la_debug_block", "la_debug_window", "la_debug_pool",
    "la_debug_pool_insert", "la_debug_kv", "la_debug_state",
    "la_attention_workspace_bytes", "la_attention", "la_attention_noalloc", "la_profile_step",
    "la_profile_kernel", "la_seed_pool", "la_prefill_seq", "la_seed_pool_seq",
    "la_debug_pool_insert_seq", "la_set_sampling", "la_sample",
]

PROF_CLASSES = ["qkv", "attention", "o_proj", "gate_up", "down", "lm_head",
                "reduce", "other"]


class LaConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float),
                ("rms_eps", C.c_float), ("W", C.c_int32), ("N", C.c_int32),
                ("G", C.c_int32), ("max_ctx", C.c_int32),
                ("dtype", C.c_int32), ("batch", C.c_int32)]


class LaStepResult(C.Structure):
    _fields_ = [("n_emitted", C.c_int32), ("tokens", C.c_int32 * 32),
                ("accepted", C.c_int32), ("winner", C.c_int32),
                ("n_candidates", C.c_int32), ("kv_len", C.c_int32)]


class LaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load liblaamd.so (building it first if it is not there)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
        pi = C.POINTER(C.c_int32)
        pf = C.POINTER(C.c_float)
        sig = {
            "la_workspace_bytes": (SZ, [C.POINTER(LaConfig)]),
            "la_create": (C.c_int, [C.POINTER(LaConfig), C.POINTER(C.c_void_p), P, SZ, P,
                                    C.POINTER(C.c_void_p)]),
            "la_prefill": (C.c_int, [P, pi, I32, pi, pi]),
            "la_step": (C.c_int, [P, C.POINTER(LaStepResult)]),
            "la_step_submit": (C.c_int, [P]),
            "la_step_collect": (C.c_int, [P, C.POINTER(LaStepResult)]),
            "la_destroy": (C.c_int, [P]),
            "la_status_string": (C.c_char_p, [C.c_int]),
            "la_last_error": (C.c_char_p, [P]),
            "la_step_rows": (I32, [P]),
            "la_debug_logits": (C.c_int, [P, pf, SZ]),
            "la_debug_block": (C.c_int, [P, pi, pi]),
            "la_debug_window": (C.c_int, [P, pi]),
            "la_debug_pool": (C.c_int, [P, pi, pi]),
            "la_debug_pool_insert": (C.c_int, [P, I32, pi]),
            "la_debug_kv": (C.c_int, [P, I32, I32, I32, pf, pf]),
            "la_debug_state": (C.c_int, [P, pi, pi]),
            "la_attention_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
            "la_attention": (C.c_int, [P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                       I32, P, SZ, P]),
            "la_attention_noalloc": (C.c_int, [P, P, P, P, I32, I32, I32, I32, I32, I32,
                                               I32, I32, P]),
            "la_profile_step": (C.c_int, [P, pf, pi, C.POINTER(LaStepResult)]),
            "la_profile_kernel": (C.c_int, [P, I32, I32, pf]),
            "la_seed_pool": (C.c_int, [P, pi, I32]),
            "la_prefill_seq": (C.c_int, [P, I32, pi, I32, pi, pi]),
            "la_seed_pool_seq": (C.c_int, [P, I32, pi, I32]),
            "la_debug_pool_insert_seq": (C.c_int, [P, I32, I32, pi]),
            "la_set_sampling": (C.c_int, [P, I32, C.c_float, I32, C.c_float, C.c_uint64]),
            "la_sample": (C.c_int, [P, I32, I32, C.c_float, I32, C.c_float, C.c_uint64, P, P,
                                    P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def make_config(cfg, max_ctx: int, batch: int = 1) -> LaConfig:
    """la_config from an object with the model fields (e.g. a lasynth config)."""
    return LaConfig(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads,
                    cfg.head_dim, cfg.d_ffn, cfg.vocab, cfg.rope_theta,
                    cfg.rms_eps, cfg.W, cfg.N, cfg.G, max_ctx,
                    LA_BF16 if cfg.dtype == "bf16" else LA_F32, batch)


def workspace_bytes(cfg, max_ctx: int, batch: int = 1) -> int:
    c = make_config(cfg, max_ctx, batch)
    return int(lib().la_workspace_bytes(C.byref(c)))


def _result(r) -> dict:
    n = int(r.n_emitted)
    return dict(n_emitted=n, tokens=[int(x) for x in r.tokens[:n]],
                accepted=int(r.accepted), winner=int(r.winner),
                n_candidates=int(r.n_candidates), kv_len=int(r.kv_len))


def upload_weights(weights, device="cuda"):
    """Host arrays (float32, or uint16 bfloat16 bit patterns) to device
    tensors, unchanged bit for bit."""
    import torch
    out = []
    for a in weights:
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
        out.append(t)
    return out


class LookaheadDecoder:
    """One decoding context (la_create ... la_destroy) of `batch` sequences.

    With batch == 1 every call speaks of the one sequence (step() returns a
    dict, the inspection calls arrays without a sequence axis); with batch >
    1 step() returns one dict per sequence and the inspection calls add a
    leading sequence axis."""

    def __init__(self, cfg, dev_weights, max_ctx: int, stream=None, batch: int = 1):
        import torch
        self.cfg = cfg
        self.max_ctx = max_ctx
        self.B = int(batch)
        self._c = make_config(cfg, max_ctx, self.B)
        L = lib()
        n = int(L.la_workspace_bytes(C.byref(self._c)))
        if n == 0:
            raise LaError(LA_ERR_INVALID_ARG, "invalid configuration")
        self.workspace = torch.empty(n, dtype=torch.uint8, device="cuda")
        self._weights = list(dev_weights)  # keep alive
        ptrs = (C.c_void_p * len(self._weights))(
            *[t.data_ptr() for t in self._weights])
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        h = C.c_void_p()
        st = L.la_create(C.byref(self._c), ptrs, self.workspace.data_ptr(), n,
                         self.stream.cuda_stream, C.byref(h))
        if st != LA_OK:
            msg = L.la_last_error(h).decode() if h.value else ""
            if h.value:
                L.la_destroy(h)
            raise LaError(st, "la_create failed: " +
                          L.la_status_string(st).decode() + " " + msg)
        self._h = h
        self.T = int(L.la_step_rows(h))

    def _check(self, st, what):
        if st != LA_OK:
            raise LaError(st, f"{what}: {lib().la_status_string(st).decode()}: "
                              f"{lib().la_last_error(self._h).decode()}")

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().la_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, prompt, init_window=None, seq: int = 0) -> int:
        """Prefill sequence seq; returns its first generated token."""
        pa, pp = _i32(prompt)
        wp = None
        if init_window is not None:
            wa, wp = _i32(init_window)
        first = C.c_int32()
        self._check(lib().la_prefill_seq(self._h, int(seq), pp, len(pa), wp, C.byref(first)),
                    "la_prefill_seq")
        return int(first.value)

    def _squeeze(self, out):
        return out[0] if self.B == 1 else out

    def step(self):
        r = (LaStepResult * self.B)()
        self._check(lib().la_step(self._h, r), "la_step")
        return self._squeeze([_result(x) for x in r])

    def step_submit(self) -> None:
        """Enqueue the next step without waiting (at most two in flight)."""
        self._check(lib().la_step_submit(self._h), "la_step_submit")

    def step_collect(self):
        """Wait for the oldest submitted step; its results, as step() returns them."""
        r = (LaStepResult * self.B)()
        self._check(lib().la_step_collect(self._h, r), "la_step_collect")
        return self._squeeze([_result(x) for x in r])

    def profile_step(self):
        """One step with per-launch HIP event timing: (result, {class: (ms, launches)})."""
        r = (LaStepResult * self.B)()
        ms = (C.c_float * len(PROF_CLASSES))()
        n = (C.c_int32 * len(PROF_CLASSES))()
        self._check(lib().la_profile_step(self._h, ms, n, r), "la_profile_step")
        res = self._squeeze([_result(x) for x in r])
        return res, {c: (float(ms[i]), int(n[i])) for i, c in enumerate(PROF_CLASSES)}

    def set_sampling(self, temperature: float, top_k: int = 0, top_p: float = 1.0,
                     seed: int = 0, seq: int = 0) -> None:
        """Draw sequence seq's tokens (temperature > 0) instead of taking the
        argmax; temperature 0 returns to greedy decoding (la_set_sampling)."""
        self._check(lib().la_set_sampling(self._h, int(seq), float(temperature), int(top_k),
                                          float(top_p), int(seed) & (2**64 - 1)),
                    "la_set_sampling")

    def seed_pool(self, tokens, seq: int = 0) -> None:
        """Insert every N-gram of tokens (e.g. the prompt) into sequence
        seq's pool, in position order; call after that sequence's prefill."""
        a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        self._check(lib().la_seed_pool_seq(self._h, int(seq),
                                           a.ctypes.data_as(C.POINTER(C.c_int32)), len(a)),
                    "la_seed_pool_seq")

    def profile_kernel(self, klass: str, reps: int = 32) -> float:
        """Mean microseconds per launch of one kernel class, from reps
        back-to-back launches between two HIP events; launch i uses layer
        (i mod n_layers)'s weights, so no launch finds its weights cached."""
        us = C.c_float()
        self._check(lib().la_profile_kernel(self._h, PROF_CLASSES.index(klass), int(reps),
                                            C.byref(us)), "la_profile_kernel")
        return float(us.value)

    def generate(self, prompt, init_window, M: int):
        if self.B != 1:
            raise ValueError("generate() drives a single-sequence decoder")
        out = [self.prefill(prompt, init_window)]
        steps = []
        while len(out) < M:
            r = self.step()
            steps.append(r)
            out += r["tokens"]
        return out[:M], steps

    # -- inspection -------------------------------------------------------
    def debug_logits(self) -> np.ndarray:
        """[batch * T][vocab]: sequence b's rows are b*T .. b*T + T - 1."""
        a = np.zeros((self.B * self.T, self.cfg.vocab), np.float32)
        self._check(lib().la_debug_logits(self._h, a.ctypes.data_as(C.POINTER(C.c_float)),
                                          a.size), "la_debug_logits")
        return a

    def debug_block(self):
        t = np.zeros(self.B * self.T, np.int32)
        a = np.zeros(self.B * self.T, np.int32)
        self._check(lib().la_debug_block(self._h, _i32(t)[1], _i32(a)[1]), "la_debug_block")
        return t, a

    def debug_window(self) -> np.ndarray:
        w = np.zeros((self.B, self.cfg.N - 1, self.cfg.W), np.int32)
        if self.cfg.W:
            self._check(lib().la_debug_window(self._h, w.ctypes.data_as(C.POINTER(C.c_int32))),
                        "la_debug_window")
        return self._squeeze(w)

    def debug_pool(self):
        c = self.cfg
        pi = C.POINTER(C.c_int32)
        ln = np.zeros((self.B, c.vocab), np.int32)
        tl = np.zeros((self.B, c.vocab, max(c.G, 1), c.N - 1), np.int32)
        self._check(lib().la_debug_pool(self._h, ln.ctypes.data_as(pi), tl.ctypes.data_as(pi)),
                    "la_debug_pool")
        if self.B == 1:
            return ln[0], tl[0, :, :c.G]
        return ln, tl[:, :, :c.G]

    def debug_pool_insert(self, key: int, tail, seq: int = 0) -> None:
        ta, tp = _i32(tail)
        self._check(lib().la_debug_pool_insert_seq(self._h, int(seq), int(key), tp),
                    "la_debug_pool_insert_seq")

    def debug_kv(self, layer: int, pos0: int, n: int):
        c = self.cfg
        k = np.zeros((self.B, c.n_kv_heads, n, c.head_dim), np.float32)
        v = np.zeros_like(k)
        pf = C.POINTER(C.c_float)
        self._check(lib().la_debug_kv(self._h, layer, pos0, n, k.ctypes.data_as(pf),
                                      v.ctypes.data_as(pf)), "la_debug_kv")
        return self._squeeze(k), self._squeeze(v)

    def debug_state(self):
        """(kv_len, current token), per sequence when batch > 1."""
        pi = C.POINTER(C.c_int32)
        L = np.zeros(self.B, np.int32)
        cur = np.zeros(self.B, np.int32)
        self._check(lib().la_debug_state(self._h, L.ctypes.data_as(pi), cur.ctypes.data_as(pi)),
                    "la_debug_state")
        return self._squeeze([(int(a), int(b)) for a, b in zip(L, cur)])


def sample(logits, temperature, top_k, top_p, seed, positions, out=None, stream=None):
    """One draw per row of device logits [rows][vocab] (fp32) with the
    uniform of positions[r] (device int64); returns out (device int32)."""
    import torch
    rows, vocab = int(logits.shape[0]), int(logits.shape[1])
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    st = lib().la_sample(logits.data_ptr(), rows, vocab, float(temperature), int(top_k),
                         float(top_p), int(seed) & (2**64 - 1), positions.data_ptr(),
                         out.data_ptr(), s.cuda_stream)
    if st != LA_OK:
        raise LaError(st, "la_sample: " + lib().la_status_string(st).decode())
    return out


def attention(q, k_cache, vt_cache, out, n_heads, n_kv_heads, prefix_len, W, N, G,
              workspace=None, stream=None):
    """One layer's masked attention (la_attention) on device tensors.

    q [rows][H][128] bf16, k_cache [Hkv][ctx][128] bf16, vt_cache
    [Hkv][128][ctx] bf16, out [rows][H][128] bf16 (written)."""
    import torch
    L = lib()
    ctx = int(k_cache.shape[1])
    need = int(L.la_attention_workspace_bytes(n_heads, 128, ctx, W, N, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    st = L.la_attention(q.data_ptr(), k_cache.data_ptr(), vt_cache.data_ptr(),
                        out.data_ptr(), n_heads, n_kv_heads, 128, prefix_len, ctx,
                        W, N, G, workspace.data_ptr(), workspace.numel(),
                        s.cuda_stream)
    if st != LA_OK:
        raise LaError(st, "la_attention: " + L.la_status_string(st).decode())
    return out


def attention_noalloc(q, k_cache, vt_cache, out, n_heads, n_kv_heads, prefix_len, W, N, G,
                      stream=None):
    """la_attention_noalloc: as attention(), with the library's own device
    scratch array instead of a workspace (nothing is allocated)."""
    import torch
    L = lib()
    ctx = int(k_cache.shape[1])
    s = stream if stream is not None else torch.cuda.current_stream()
    st = L.la_attention_noalloc(q.data_ptr(), k_cache.data_ptr(), vt_cache.data_ptr(),
                                out.data_ptr(), n_heads, n_kv_heads, 128, prefix_len, ctx,
                                W, N, G, s.cuda_stream)
    if st != LA_OK:
        raise LaError(st, "la_attention_noalloc: " + L.la_status_string(st).decode())
    return out
