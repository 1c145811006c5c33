"""Seeded synthetic inputs for the verification step.

This module makes logits and drafted tokens; it holds none of the
verification rule.  Both the library's tests and benchmark and the oracle's
tests draw their inputs from here, so that both sides see the same stored
tensors (the stored bits are the truth for both).

Workloads (B sequences, gamma drafts, vocabulary V):

  c0   B=1,    gamma=4, V=256,    fp32, target N(0, 3^2), draft = target + N(0, 1),  T=1
  c1   B=8,    gamma=3, V=32000,  fp32, target N(0, 2.5^2), draft = 0.9 target + N(0, 1.5^2), T=1
  c2   B=64,   gamma=5, V=128256, bf16, target N(0, 3^2) + Zipf(1.1) bias, draft = target + N(0, 1), T=0.7
  c3   B=256,  gamma=8, V=152064, bf16, as c2 with draft noise sigma 2, T=0.8, top-k 50
  c4a/b/c B=1024, gamma=4, V=50257, fp32, target N(0, 3^2), draft = target + N(0, s^2),
       s = 0.25 / 1 / 4, T=1
  c3p  c3 with top-p 0.9 after the top-k 50 (nucleus)
  c2p  c2 with top-p 0.9 and no top-k (nucleus over the whole vocabulary)
  g2   c2's logits at T=0 (arg-max mode)
  g4b  c4b's logits at T=0 (arg-max mode)

The Zipf bias of a target row is -1.1 * ln(rank), rank = pi(v) + 1 for a fresh
uniform permutation pi of the vocabulary per target row; a draft row inherits
the bias of the target row at the same position through "draft = target +
noise".  bf16 logits are rounded from fp32 to nearest-even.

Drafted tokens stand in for the draft model's own sampling (outside the
verification step): token j of a sequence is drawn from the draft row's
adjusted distribution softmax(top-k(z) / T) by inverse CDF with a numpy
generator; at T=0 it is the draft row's first largest logit.  The top-k here keeps the K largest logits, the smaller index on
equal logits, so drafted tokens lie inside the draft's kept set.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

ZIPF_S = 1.1


@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    gamma: int
    V: int
    dtype: str              # "f32" | "bf16"
    temperature: float
    top_k: int
    target_sigma: float
    draft_scale: float      # draft = draft_scale * target + N(0, draft_sigma^2)
    draft_sigma: float
    zipf: bool
    data_seed: int
    draft_seed: int
    top_p: float = 1.0       # nucleus mass (1: off)


SPECS = {
    "c0": Spec("c0", 1, 4, 256, "f32", 1.0, 0, 3.0, 1.0, 1.0, False, 1000, 2000),
    "c1": Spec("c1", 8, 3, 32000, "f32", 1.0, 0, 2.5, 0.9, 1.5, False, 1001, 2001),
    "c2": Spec("c2", 64, 5, 128256, "bf16", 0.7, 0, 3.0, 1.0, 1.0, True, 1002, 2002),
    "c3": Spec("c3", 256, 8, 152064, "bf16", 0.8, 50, 3.0, 1.0, 2.0, True, 1003, 2003),
    "c4a": Spec("c4a", 1024, 4, 50257, "f32", 1.0, 0, 3.0, 1.0, 0.25, False, 1040, 2040),
    "c4b": Spec("c4b", 1024, 4, 50257, "f32", 1.0, 0, 3.0, 1.0, 1.0, False, 1041, 2041),
    "c4c": Spec("c4c", 1024, 4, 50257, "f32", 1.0, 0, 3.0, 1.0, 4.0, False, 1042, 2042),
    "c3p": Spec("c3p", 256, 8, 152064, "bf16", 0.8, 50, 3.0, 1.0, 2.0, True, 1003, 2003, 0.9),
    "c2p": Spec("c2p", 64, 5, 128256, "bf16", 0.7, 0, 3.0, 1.0, 1.0, True, 1002, 2002, 0.9),
    "g2": Spec("g2", 64, 5, 128256, "bf16", 0.0, 0, 3.0, 1.0, 1.0, True, 1002, 2002),
    "g4b": Spec("g4b", 1024, 4, 50257, "f32", 0.0, 0, 3.0, 1.0, 1.0, False, 1041, 2041),
}


@dataclass
class Workload:
    spec: Spec
    target: np.ndarray      # [B, gamma+1, V] float32, or uint16 bf16 bits
    draft: np.ndarray       # [B, gamma, V]   same dtype as target
    tokens: np.ndarray      # [B, gamma] int32

    @property
    def B(self): return self.target.shape[0]
    @property
    def gamma(self): return self.draft.shape[1]
    @property
    def V(self): return self.target.shape[2]
    @property
    def temperature(self): return self.spec.temperature
    @property
    def top_k(self): return self.spec.top_k
    @property
    def top_p(self): return self.spec.top_p
    @property
    def is_bf16(self): return self.target.dtype == np.uint16

    def nbytes(self) -> int:
        return self.target.nbytes + self.draft.nbytes + self.tokens.nbytes


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def logits_f32(a: np.ndarray) -> np.ndarray:
    """Stored logits as float32 (exact for both storage types)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


# ---------------------------------------------------------------------------
# Draft-token sampler (stand-in for the draft model)
# ---------------------------------------------------------------------------
def _adjusted(z: np.ndarray, temperature: float, top_k: int, top_p: float = 1.0) -> np.ndarray:
    """Rows of z [R, V] float64 -> softmax(top-k(z) / T), then the nucleus of
    mass top_p in the same order (larger logit, then smaller index), as
    float64 [R, V]."""
    R, V = z.shape
    x = z / float(np.float32(temperature))
    order = np.argsort(-z, axis=1, kind="stable")
    if 0 < top_k < V:
        mask = np.zeros_like(z, dtype=bool)
        np.put_along_axis(mask, order[:, :top_k], True, axis=1)
        x = np.where(mask, x, -np.inf)
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    p = e / e.sum(axis=1, keepdims=True)
    P = float(np.float32(top_p))
    if 0 < P < 1:
        ps = np.take_along_axis(p, order, axis=1)
        cum = np.cumsum(ps, axis=1)
        keep_sorted = (cum - ps) < P          # entries before the one that reaches P, and it
        keep = np.zeros_like(keep_sorted)
        np.put_along_axis(keep, order, keep_sorted, axis=1)
        p = np.where(keep, p, 0.0)
        p = p / p.sum(axis=1, keepdims=True)
    return p


def sample_rows(z: np.ndarray, temperature: float, top_k: int, rng: np.random.Generator,
                chunk: int = 256, top_p: float = 1.0) -> np.ndarray:
    """One token per row of z [R, V] from the row's adjusted distribution
    (T = 0: the first largest logit)."""
    R, V = z.shape
    if temperature == 0.0:
        return np.argmax(np.asarray(z), axis=1).astype(np.int32)
    out = np.empty(R, dtype=np.int32)
    for s in range(0, R, chunk):
        p = _adjusted(np.asarray(z[s:s + chunk], dtype=np.float64), temperature, top_k, top_p)
        cdf = np.cumsum(p, axis=1)
        u = rng.random(p.shape[0]) * cdf[:, -1]
        t = (cdf <= u[:, None]).sum(axis=1)
        t = np.minimum(t, V - 1)
        # never land on a zero-probability entry (possible only at float ties of the cdf)
        bad = p[np.arange(p.shape[0]), t] == 0.0
        if bad.any():
            t[bad] = np.argmax(p[bad], axis=1)
        out[s:s + chunk] = t
    return out


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
def _zipf_bias_row(V: int, rng: np.random.Generator) -> np.ndarray:
    ranks = rng.permutation(V).astype(np.float64) + 1.0
    return (-ZIPF_S * np.log(ranks)).astype(np.float32)


def make(name: str, B: int | None = None, data_seed: int | None = None,
         draft_seed: int | None = None, **overrides) -> Workload:
    """Build workload `name`; B and the seeds may be overridden (the first B
    sequences of the full workload are the same whatever B is)."""
    spec = SPECS[name]
    if B is not None:
        spec = replace(spec, B=B)
    if data_seed is not None:
        spec = replace(spec, data_seed=data_seed)
    if draft_seed is not None:
        spec = replace(spec, draft_seed=draft_seed)
    if overrides:
        spec = replace(spec, **overrides)
    return build(spec)


def build(spec: Spec) -> Workload:
    B, g, V = spec.B, spec.gamma, spec.V
    rng = np.random.default_rng(spec.data_seed)
    store = np.uint16 if spec.dtype == "bf16" else np.float32
    target = np.empty((B, g + 1, V), dtype=store)
    draft = np.empty((B, g, V), dtype=store)
    for b in range(B):  # per sequence, so a prefix of B is stable
        t = rng.standard_normal((g + 1, V), dtype=np.float32) * np.float32(spec.target_sigma)
        if spec.zipf:
            for j in range(g + 1):
                t[j] += _zipf_bias_row(V, rng)
        noise = rng.standard_normal((g, V), dtype=np.float32) * np.float32(spec.draft_sigma)
        d = np.float32(spec.draft_scale) * t[:g] + noise
        if store is np.uint16:
            target[b] = f32_to_bf16_bits(t)
            draft[b] = f32_to_bf16_bits(d)
        else:
            target[b] = t
            draft[b] = d
    drng = np.random.default_rng(spec.draft_seed)
    z = logits_f32(draft.reshape(B * g, V))
    tokens = sample_rows(z, spec.temperature, spec.top_k, drng, top_p=spec.top_p).reshape(B, g)
    return Workload(spec, target, draft, tokens)


def replicate_position(w: Workload, b: int, j: int, n_seq: int, seed: int) -> Workload:
    """n_seq one-draft sequences that all verify position (b, j) of w: target rows
    (q_j, q_j), draft row p_j, each token drawn afresh from p_j."""
    V = w.V
    q = w.target[b, j]
    p = w.draft[b, j]
    target = np.broadcast_to(q, (n_seq, 2, V)).copy()
    draft = np.broadcast_to(p, (n_seq, 1, V)).copy()
    rng = np.random.default_rng(seed)
    probs = _adjusted(logits_f32(p[None, :]).astype(np.float64), w.temperature, w.top_k)[0]
    cdf = np.cumsum(probs)
    u = rng.random(n_seq) * cdf[-1]
    tok = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)
    spec = replace(w.spec, name=f"{w.spec.name}-pos{b}.{j}x{n_seq}", B=n_seq, gamma=1)
    return Workload(spec, target, draft, tok.reshape(n_seq, 1))


def from_arrays(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray,
                temperature: float = 1.0, top_k: int = 0, name: str = "custom", top_p: float = 1.0) -> Workload:
    B, g1, V = target.shape
    spec = Spec(name, B, g1 - 1, V, "bf16" if target.dtype == np.uint16 else "f32",
                temperature, top_k, 0.0, 0.0, 0.0, False, -1, -1, top_p)
    return Workload(spec, np.ascontiguousarray(target), np.ascontiguousarray(draft),
                    np.ascontiguousarray(tokens, dtype=np.int32))


# ---------------------------------------------------------------------------
# Token-dependent rows: a first-order Markov "model" pair
# ---------------------------------------------------------------------------
@dataclass
class MarkovPair:
    """Logit tables of a target and a draft model whose next-token logits
    depend on the previous token only: row x of `target` ([V, V] float32) is
    the target's logits after token x, row x of `draft` the draft's."""
    target: np.ndarray
    draft: np.ndarray

    @property
    def V(self):
        return self.target.shape[0]


def markov_pair(V: int = 64, target_sigma: float = 3.0, draft_sigma: float = 1.0, seed: int = 1077) -> MarkovPair:
    """Target table N(0, target_sigma^2); draft table = target + N(0, draft_sigma^2)."""
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((V, V), dtype=np.float32) * np.float32(target_sigma)).astype(np.float32)
    d = (t + rng.standard_normal((V, V), dtype=np.float32) * np.float32(draft_sigma)).astype(np.float32)
    return MarkovPair(t, d)
