"""Seeded synthetic inputs for the MoE dispatch / grouped-FFN / combine path.

This module only *draws* inputs. It holds none of the layer's arithmetic, so
both the CPU oracle (through the tests and the bench's baseline leg) and the
GPU path can take their inputs from here without sharing any method code.

Storage conventions
-------------------
* fp32 tensors are ``numpy.float32`` arrays.
* bf16 tensors are ``numpy.uint16`` arrays holding the bf16 bit patterns. They
  are produced from fp32 draws by round-to-nearest-even on the upper 16 bits.
* Every array is C-contiguous and row-major. Weights use the ``[out, in]``
  convention, so a product is ``x @ W.T``.

Workloads
---------
The pages only say that MoE training was run on packed 32k-token sequences at
DP4/EP2 and DP4/EP4 ("Add MoE expert parallel training runtime", author
comment). They print no data, so every value here is synthetic. A 32k-token
microbatch stands for one packed sequence held by one expert-parallel rank,
routed over that rank's local experts only.

Draw order from ``numpy.random.Generator(PCG64(seed))``: x, w_router, w_gu,
w_down, routing-logit noise, dout. Weights are N(0, 0.02^2) (0.02 is the
standard deviation).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# bf16 storage helpers (representation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    NaN inputs are not expected from the generators; they are mapped to a
    quiet NaN pattern so that they stay NaN.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (the largest,
    # -inf = 0xFF800000, gains at most 0x8000); NaNs are overwritten below
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    r = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored tensor (fp32 array or bf16 bits) to fp64 exactly."""
    if dtype == BF16 and a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 draws to the storage type of ``dtype``."""
    a = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a)


# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int                     # tokens (single microbatch) -- see ``micro_T``
    d: int
    E: int
    k: int
    F: int
    dtype: str
    routing: str               # "router" | "zipf" | "normal"
    x_std: float = 1.0
    zipf_s: float = 0.0
    n_empty: int = 0           # experts forced empty
    micro_T: Optional[tuple] = None   # microbatch token counts (accumulation run)
    renorm: bool = False
    description: str = ""

    @property
    def microbatches(self) -> tuple:
        return self.micro_T if self.micro_T is not None else (self.T,)

    def flops_fwd(self, T: Optional[int] = None) -> float:
        """Algorithmic FLOPs of one forward pass (grouped GEMMs, plus the
        router GEMM when it runs)."""
        ts = (T,) if T is not None else self.microbatches
        fl = 0.0
        for t in ts:
            fl += 6.0 * t * self.k * self.d * self.F
            if self.routing == "router":
                fl += 2.0 * t * self.d * self.E
        return fl

    def flops_fwd_bwd(self, T: Optional[int] = None) -> float:
        """Algorithmic FLOPs of one forward+backward pass (grouped GEMMs only,
        plus the router GEMM when it runs)."""
        ts = (T,) if T is not None else self.microbatches
        fl = 0.0
        for t in ts:
            R = t * self.k
            fl += 18.0 * R * self.d * self.F
            if self.routing == "router":
                fl += 6.0 * t * self.d * self.E
        return fl


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 64, 64, 4, 2, 128, F32, "router", x_std=0.02,
                 description="tiny fp32 layer: T=64 d=64 E=4 top-2 F=128, router GEMM"),
        Workload("router_bf16", 2, 4096, 1024, 8, 2, 2816, BF16, "router", n_empty=1,
                 description="bf16 T=4096 d=1024 E=8 top-2 F=2816, router bias empties one expert"),
        Workload("ep_share_32k", 3, 32768, 2048, 32, 8, 1408, BF16, "zipf", zipf_s=1.2, n_empty=2,
                 description="one EP rank's share of a packed 32k sequence: T=32768 d=2048 "
                             "E_local=32 top-8 F=1408, Zipf(1.2) popularity, 2 experts empty"),
        Workload("microbatches_32k", 4, 32768, 2048, 32, 8, 1408, BF16, "zipf", zipf_s=1.2,
                 n_empty=2, micro_T=(16384, 7001, 0, 32768),
                 description="4 microbatches T in {16384,7001,0,32768}, d=2048 E_local=32 top-8 "
                             "F=1408, fp32 dW accumulated across microbatches"),
        Workload("large_share_uniform", 5, 32768, 4096, 64, 8, 1536, BF16, "normal",
                 description="T=32768 d=4096 E_local=64 top-8 F=1536, logits N(0,1)"),
        Workload("large_share_zipf", 6, 32768, 4096, 64, 8, 1536, BF16, "zipf", zipf_s=1.0,
                 description="T=32768 d=4096 E_local=64 top-8 F=1536, Zipf(1.0) popularity"),
    ]
}


def small_workload(T: int, d: int, E: int, k: int, F: int, dtype: str = BF16, routing: str = "normal",
                   seed: int = 11, zipf_s: float = 1.2, n_empty: int = 0, renorm: bool = False,
                   x_std: float = 1.0, micro_T: Optional[tuple] = None) -> Workload:
    """An ad-hoc workload for edge-case tests."""
    return Workload(f"adhoc_T{T}_d{d}_E{E}_k{k}_F{F}_{dtype}_{routing}", seed, T, d, E, k, F, dtype,
                    routing, x_std=x_std, zipf_s=zipf_s, n_empty=n_empty, micro_T=micro_T,
                    renorm=renorm)


# --------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _zipf_logits(rng: np.random.Generator, T: int, E: int, s: float, n_empty: int) -> np.ndarray:
    """log(popularity) + Gumbel(0,1) noise, popularity ~ rank^-s over the
    non-empty experts (ranks mapped to ids by a seeded permutation); forced-empty
    experts get logit -1e4. The top-k of such logits is a draw of k distinct
    experts without replacement, in proportion to popularity (Gumbel-top-k)."""
    perm = rng.permutation(E)
    empty = perm[:n_empty]
    live = perm[n_empty:]
    pop = np.zeros(E, dtype=np.float64)
    ranks = np.arange(1, len(live) + 1, dtype=np.float64)
    pop[live] = ranks ** (-s)
    pop /= pop.sum()
    logp = np.full(E, -1e4, dtype=np.float64)
    logp[live] = np.log(pop[live])
    g = rng.gumbel(size=(T, E)).astype(np.float32)
    logits = (logp.astype(np.float32)[None, :] + g).astype(np.float32)
    logits[:, empty] = np.float32(-1e4)
    return np.ascontiguousarray(logits)


def make_weights(w: Workload, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    out = {}
    if w.routing == "router":
        out["w_router"] = store(_normal(rng, (w.E, w.d), 0.02), w.dtype)
        bias = np.zeros(w.E, dtype=np.float32)
        if w.n_empty:
            bias[rng.permutation(w.E)[: w.n_empty]] = np.float32(-1e4)
        out["bias"] = bias
    out["w_gu"] = store(_normal(rng, (w.E, 2 * w.F, w.d), 0.02), w.dtype)
    out["w_down"] = store(_normal(rng, (w.E, w.d, w.F), 0.02), w.dtype)
    return out


def make_microbatch(w: Workload, T: int, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    out = {"x": store(_normal(rng, (T, w.d), w.x_std), w.dtype)}
    if w.routing == "zipf":
        out["logits"] = _zipf_logits(rng, T, w.E, w.zipf_s, w.n_empty)
    elif w.routing == "normal":
        out["logits"] = _normal(rng, (T, w.E), 1.0)
    out["dout"] = store(_normal(rng, (T, w.d), 1.0), w.dtype)
    return out


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, object]:
    """All inputs of a workload.

    Returns ``{"weights": {...}, "micro": [ {x, logits?, dout}, ... ]}``; one
    entry of ``micro`` per microbatch (a single one for a plain workload).
    Draw order: x of the first microbatch, then the weights, then the routing
    noise and dout of the first microbatch; later microbatches draw x, noise
    and dout in turn from the same stream.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    ts = w.microbatches
    x0 = store(_normal(rng, (ts[0], w.d), w.x_std), w.dtype)
    weights = make_weights(w, rng)
    micro: List[Dict[str, np.ndarray]] = []
    for i, T in enumerate(ts):
        if i == 0:
            mb = {"x": x0}
            if w.routing == "zipf":
                mb["logits"] = _zipf_logits(rng, T, w.E, w.zipf_s, w.n_empty)
            elif w.routing == "normal":
                mb["logits"] = _normal(rng, (T, w.E), 1.0)
            mb["dout"] = store(_normal(rng, (T, w.d), 1.0), w.dtype)
        else:
            mb = make_microbatch(w, T, rng)
        micro.append(mb)
    return {"weights": weights, "micro": micro}


def make_ep_inputs(ep: int, Ts, d: int, e_local: int, k: int, F: int, dtype: str = BF16, seed: int = 0,
                   routing: str = "normal", zipf_s: float = 1.2, n_empty: int = 0) -> Dict[str, object]:
    """Inputs of EP ranks simulated together: weights of all ep * e_local
    experts, and per source rank its tokens x [T_s, d], routing logits
    [T_s, E] (N(0,1), or Zipf popularity over the global experts with n_empty
    experts forced empty, the same popularity on every rank) and dout.
    Draw order: weights, then per source x, logits noise, dout."""
    E = ep * e_local
    w = Workload(f"ep{ep}", seed, max(Ts) if len(Ts) else 0, d, E, k, F, dtype, routing, zipf_s=zipf_s,
                 n_empty=n_empty)
    rng = np.random.Generator(np.random.PCG64(seed))
    weights = make_weights(w, rng)
    perm = rng.permutation(E) if routing == "zipf" else None
    micro = []
    for T in Ts:
        x = store(_normal(rng, (T, d), 1.0), dtype)
        if routing == "zipf":
            empty, live = perm[:n_empty], perm[n_empty:]
            pop = np.zeros(E)
            pop[live] = np.arange(1, len(live) + 1, dtype=np.float64) ** (-zipf_s)
            logp = np.full(E, -1e4)
            logp[live] = np.log(pop[live] / pop.sum())
            lg = (logp.astype(np.float32)[None, :] + rng.gumbel(size=(T, E)).astype(np.float32)).astype(np.float32)
            lg[:, empty] = np.float32(-1e4)
        else:
            lg = _normal(rng, (T, E), 1.0)
        micro.append({"x": x, "logits": np.ascontiguousarray(lg), "dout": store(_normal(rng, (T, d), 1.0), dtype)})
    return {"weights": weights, "micro": micro}


def tie_logits(T: int, E: int, seed: int, levels: int = 3) -> np.ndarray:
    """fp32 logits drawn from a handful of integer levels, so that most tokens
    hold ties (used to exercise the lowest-id tie-break)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, levels, size=(T, E)).astype(np.float32)


def flops_per_routed_row(d: int, F: int) -> float:
    """6*d*F forward + 12*d*F backward per routed (token, expert) row."""
    return 18.0 * d * F


def describe(w: Workload) -> str:
    return w.description or w.name


__all__ = [
    "F32", "BF16", "Workload", "WORKLOADS", "small_workload", "make_inputs", "make_weights",
    "make_microbatch", "make_ep_inputs", "tie_logits", "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f64", "store",
    "flops_per_routed_row", "describe",
]
