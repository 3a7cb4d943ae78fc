"""ctypes wrapper of the CPU oracle (``la_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.  It
shares no code with the HIP library.

The oracle computes in float64 with a fixed reduction order (see the C
source header for the method and every reading of the pages it takes).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liblaoracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into oracle/_build/liblaoracle.so."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Cfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_double),
                ("rms_eps", C.c_double), ("W", C.c_int32), ("N", C.c_int32),
                ("G", C.c_int32), ("max_ctx", C.c_int32),
                ("wdtype", C.c_int32), ("act_bf16", C.c_int32)]


class _Res(C.Structure):
    _fields_ = [("n_emitted", C.c_int32), ("tokens", C.c_int32 * 32),
                ("accepted", C.c_int32), ("winner", C.c_int32),
                ("n_candidates", C.c_int32), ("kv_len", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P, I, D = C.c_void_p, C.c_int, C.POINTER(C.c_double)
        I32 = C.POINTER(C.c_int32)
        sig = {
            "orc_create": (C.c_void_p, [C.POINTER(_Cfg), C.POINTER(C.c_void_p)]),
            "orc_destroy": (None, [P]),
            "orc_rows": (I, [P]), "orc_kv_len": (I, [P]), "orc_current": (I, [P]),
            "orc_set_threads": (None, [I]), "orc_max_threads": (I, []),
            "orc_extend": (I, [P, I32, I, D]),
            "orc_prefill": (I, [P, I32, I, I32, D]),
            "orc_block_tokens": (I, [P, I32, I32]),
            "orc_forward_block": (I, [P, I32, I32, D, I]),
            "orc_block_argmax": (I, [P, I32]),
            "orc_commit": (I, [P, I32, C.POINTER(_Res)]),
            "orc_step": (I, [P, C.POINTER(_Res), D]),
            "orc_greedy_next": (I, [P, D]),
            "orc_pool_insert": (None, [P, C.c_int32, I32]),
            "orc_seed_pool": (I, [P, I32, I]),
            "orc_get_window": (None, [P, I32]),
            "orc_set_window": (None, [P, I32]),
            "orc_set_current": (None, [P, C.c_int32]),
            "orc_get_pool": (None, [P, I32, I32]),
            "orc_get_kv": (I, [P, I, I, I, D, D]),
            "orc_row_pos": (I, [C.POINTER(_Cfg), I]),
            "orc_visible": (I, [C.POINTER(_Cfg), I, I]),
            "orc_attention": (None, [C.POINTER(_Cfg), I, P, P, P, I, I32, D]),
            "orc_philox4x32_10": (None, [C.POINTER(C.c_uint32), C.POINTER(C.c_uint32),
                                         C.POINTER(C.c_uint32)]),
            "orc_uniform": (C.c_double, [C.c_uint64, C.c_int64]),
            "orc_sample_logits": (I, [D, I, C.c_double, I, C.c_double, C.c_double, D]),
            "orc_block_select": (I, [P, I32, D]),
            "orc_set_sampling": (I, [P, C.c_double, I, C.c_double, C.c_uint64]),
            "orc_round_bf16": (C.c_double, [C.c_double]),
            "orc_rewind": (I, [P, I, C.c_int32]),
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


def _f64p(a):
    return a.ctypes.data_as(C.POINTER(C.c_double))


STORAGES = ("exact", "bf16")


def make_cfg(cfg, max_ctx: int = 0, storage: str = "exact") -> _Cfg:
    """C config from a lasynth.ModelConfig-like object.  storage: "exact"
    (no activation is rounded) or "bf16" (the seven stored activations of a
    bf16 datapath are rounded to bfloat16; see the C source header)."""
    if storage not in STORAGES:
        raise ValueError(f"storage must be one of {STORAGES}")
    return _Cfg(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads,
                cfg.head_dim, cfg.d_ffn, cfg.vocab, cfg.rope_theta,
                cfg.rms_eps, cfg.W, cfg.N, cfg.G, max_ctx,
                1 if cfg.dtype == "bf16" else 0, 1 if storage == "bf16" else 0)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def row_pos(cfg, r: int) -> int:
    c = make_cfg(cfg, 1)
    return int(lib().orc_row_pos(C.byref(c), r))


def visible(cfg, r: int, s: int) -> bool:
    c = make_cfg(cfg, 1)
    return bool(lib().orc_visible(C.byref(c), r, s))


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter and a 2-word key (4 words out)."""
    c = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (C.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def round_bf16(v: float) -> float:
    """bfloat16 storage of one value (the bf16 storage mode's rounding)."""
    return float(lib().orc_round_bf16(float(v)))


def uniform(seed: int, pos: int) -> float:
    """The uniform that draws the token at sequence position pos."""
    return float(lib().orc_uniform(int(seed) & (2**64 - 1), int(pos)))


def sample_logits(logits, temperature: float, top_k: int = 0, top_p: float = 1.0,
                  u: float = 0.5):
    """One draw from a row of logits: (token, margin); see the C source."""
    lg = np.ascontiguousarray(logits, dtype=np.float64)
    m = C.c_double()
    t = lib().orc_sample_logits(_f64p(lg), lg.size, float(temperature), int(top_k),
                                float(top_p), float(u), C.byref(m))
    return int(t), float(m.value)


def attention(cfg, L, q, k, v, bf16: bool, valid=None):
    """Masked attention of one layer (kernel-only workload); see C source."""
    c = make_cfg(cfg, 1)
    T = cfg.T
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    out = np.zeros((T, cfg.n_heads, cfg.head_dim), np.float64)
    vp = None
    if valid is not None:
        va, vp = _i32(valid)
    lib().orc_attention(C.byref(c), int(L), q.ctypes.data, k.ctypes.data,
                        v.ctypes.data, 1 if bf16 else 0, vp, _f64p(out))
    return out


class Oracle:
    """One decoding context on the CPU: KV cache, window, pool."""

    def __init__(self, cfg, weights, max_ctx: int, storage: str = "exact"):
        """storage: "exact" (default) or "bf16" activation storage."""
        self.cfg = cfg
        self.storage = storage
        self._weights = [np.ascontiguousarray(w) for w in weights]
        ptrs = (C.c_void_p * len(self._weights))(
            *[w.ctypes.data for w in self._weights])
        self._c = make_cfg(cfg, max_ctx, storage)
        self._h = lib().orc_create(C.byref(self._c), ptrs)
        if not self._h:
            raise ValueError("oracle: invalid configuration or out of memory")
        self.T = int(lib().orc_rows(self._h))
        self.max_ctx = max_ctx

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_destroy(h)
            self._h = None

    # -- state ------------------------------------------------------------
    @property
    def kv_len(self) -> int:
        return int(lib().orc_kv_len(self._h))

    @property
    def current(self) -> int:
        return int(lib().orc_current(self._h))

    def set_current(self, t: int) -> None:
        lib().orc_set_current(self._h, int(t))

    def rewind(self, L: int, cur: int) -> None:
        """Back to committed length L with current token cur (window and
        pool kept)."""
        if lib().orc_rewind(self._h, int(L), int(cur)):
            raise ValueError("bad rewind")

    def window(self) -> np.ndarray:
        c = self.cfg
        w = np.zeros((c.N - 1, c.W), np.int32)
        if c.W:
            lib().orc_get_window(self._h, _i32(w)[1])
        return w

    def set_window(self, win) -> None:
        a, p = _i32(win)
        lib().orc_set_window(self._h, p)

    def pool(self):
        c = self.cfg
        ln = np.zeros(c.vocab, np.int32)
        tl = np.zeros((c.vocab, max(c.G, 1), c.N - 1), np.int32)
        lib().orc_get_pool(self._h, _i32(ln)[1],
                           tl.ctypes.data_as(C.POINTER(C.c_int32)))
        return ln, tl[:, :c.G]

    def pool_insert(self, key: int, tail) -> None:
        a, p = _i32(tail)
        lib().orc_pool_insert(self._h, int(key), p)

    def seed_pool(self, seq) -> None:
        """Insert every N-gram of seq into the pool, in position order."""
        a, p = _i32(seq)
        if lib().orc_seed_pool(self._h, p, len(a)) != 0:
            raise ValueError("bad token sequence")

    def kv(self, layer: int, pos0: int, n: int):
        c = self.cfg
        k = np.zeros((c.n_kv_heads, n, c.head_dim), np.float64)
        v = np.zeros_like(k)
        rc = lib().orc_get_kv(self._h, layer, pos0, n, _f64p(k), _f64p(v))
        if rc:
            raise IndexError("kv range")
        return k, v

    # -- decoding ---------------------------------------------------------
    def prefill(self, prompt, init_window=None, logits: bool = False):
        pa, pp = _i32(prompt)
        wp = None
        if init_window is not None:
            wa, wp = _i32(init_window)
        lg = np.zeros((len(pa), self.cfg.vocab), np.float64) if logits else None
        t = lib().orc_prefill(self._h, pp, len(pa), wp,
                              _f64p(lg) if logits else None)
        if t < 0:
            raise ValueError("oracle prefill failed")
        return (int(t), lg) if logits else int(t)

    def extend(self, seq, logits: bool = False):
        sa, sp = _i32(seq)
        lg = np.zeros((len(sa), self.cfg.vocab), np.float64) if logits else None
        t = lib().orc_extend(self._h, sp, len(sa), _f64p(lg) if logits else None)
        if t < 0:
            raise ValueError("oracle extend failed")
        return (int(t), lg) if logits else int(t)

    def block_tokens(self):
        tok = np.zeros(self.T, np.int32)
        val = np.zeros(self.T, np.int32)
        nc = lib().orc_block_tokens(self._h, _i32(tok)[1], _i32(val)[1])
        return tok, val, int(nc)

    def forward_block(self, tok, valid, keep: bool = True):
        ta, tp = _i32(tok)
        va, vp = _i32(valid)
        lg = np.zeros((self.T, self.cfg.vocab), np.float64)
        rc = lib().orc_forward_block(self._h, tp, vp, _f64p(lg), 1 if keep else 0)
        if rc < 0:
            raise ValueError("oracle block forward failed (capacity?)")
        return lg

    def block_argmax(self) -> np.ndarray:
        a = np.zeros(self.T, np.int32)
        if lib().orc_block_argmax(self._h, _i32(a)[1]):
            raise RuntimeError("no block forwarded")
        return a

    def block_select(self):
        """Per-row decisions of the kept block (argmax for lookahead rows;
        draws for the current-token and candidate rows when sampling) and
        the draws' margins (NaN where no draw)."""
        a = np.zeros(self.T, np.int32)
        m = np.zeros(self.T, np.float64)
        if lib().orc_block_select(self._h, _i32(a)[1], _f64p(m)):
            raise RuntimeError("no block forwarded")
        return a, m

    def set_sampling(self, temperature: float, top_k: int = 0, top_p: float = 1.0,
                     seed: int = 0) -> None:
        """Draw the emitted tokens (temperature > 0) instead of the argmax."""
        if lib().orc_set_sampling(self._h, float(temperature), int(top_k), float(top_p),
                                  int(seed) & (2**64 - 1)):
            raise ValueError("bad sampling parameters")

    def commit(self, amax=None) -> dict:
        r = _Res()
        p = None
        if amax is not None:
            aa, p = _i32(amax)
        if lib().orc_commit(self._h, p, C.byref(r)):
            raise RuntimeError("no block forwarded")
        return _res_dict(r)

    def step(self, logits: bool = False):
        r = _Res()
        lg = np.zeros((self.T, self.cfg.vocab), np.float64) if logits else None
        rc = lib().orc_step(self._h, C.byref(r), _f64p(lg) if logits else None)
        if rc < 0:
            raise ValueError("oracle step failed (capacity?)")
        return (_res_dict(r), lg) if logits else _res_dict(r)

    def greedy_next(self, logits: bool = False):
        lg = np.zeros((1, self.cfg.vocab), np.float64) if logits else None
        t = lib().orc_greedy_next(self._h, _f64p(lg) if logits else None)
        if t < 0:
            raise ValueError("oracle greedy step failed (capacity?)")
        return (int(t), lg[0]) if logits else int(t)

    # -- whole runs -------------------------------------------------------
    def generate(self, prompt, init_window, M: int, seed_prompt: bool = False):
        """Lookahead decoding of M tokens (the prefill's token included);
        seed_prompt: the pool starts with the prompt's n-grams."""
        out = [self.prefill(prompt, init_window)]
        if seed_prompt:
            self.seed_pool(prompt)
        steps = []
        while len(out) < M:
            r = self.step()
            steps.append(r)
            out += r["tokens"]
        return out[:M], steps

    def greedy(self, prompt, M: int):
        """Plain one-token-at-a-time greedy decoding of M tokens."""
        out = [self.prefill(prompt, None if self.cfg.W == 0 else
                            np.zeros((self.cfg.N - 1, self.cfg.W), np.int32))]
        while len(out) < M:
            out.append(self.greedy_next())
        return out


def _res_dict(r: _Res) -> dict:
    n = int(r.n_emitted)
    return dict(n_emitted=n, tokens=[int(x) for x in r.tokens[:n]],
                accepted=int(r.accepted), winner=int(r.winner),
                n_candidates=int(r.n_candidates), kv_len=int(r.kv_len))
