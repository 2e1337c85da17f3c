"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle's tests.

This module only draws random numbers and rounds them to the storage type. It
holds none of the method's arithmetic (no pooling, scoring, selection or
attention), so both sides may import it without sharing any of the computation
under test.

Recipe (the pages publish no dataset for this path, so every input is synthetic):

* Generator: ``numpy.random.Generator(PCG64(SeedSequence([seed, workload_id, stream])))``.
  Streams: Q=1, K=2, V=3, needle direction=4, needle leaves=5, needle queries=6,
  decode q/k/v = 7/8/9.
* ``standard_normal(float32)`` values, rounded to bfloat16 (round to nearest even)
  for bf16 workloads. Layout is head-major: Q,O ``[B, Hq, N, d]``; K,V ``[B, Hkv, N, d]``.
* Keys are either i.i.d. N(0,1) or an AR(1) process along the sequence,
  k_0 = e_0, k_t = rho k_{t-1} + sqrt(1-rho^2) e_t (unit marginal variance),
  evaluated in float64 and then rounded to float32 (and bf16), independently per
  (batch, KV head).
* Planted needles (long-prefill workload): per (batch, KV head) a unit direction
  u = z/|z|; 8 leaf blocks drawn without replacement get keys 4u + N(0, 0.25 I);
  per query head, floor(0.01 N) positions drawn without replacement get queries
  3u + N(0, I).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3
STREAM_NEEDLE_DIR, STREAM_NEEDLE_LEAVES, STREAM_NEEDLE_QUERIES = 4, 5, 6
STREAM_DEC_Q, STREAM_DEC_K, STREAM_DEC_V = 7, 8, 9


def rng_for(seed: int, workload_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload_id, stream])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A host tensor in its storage type: float32 values, or bf16 bit patterns (uint16)."""

    data: np.ndarray
    dtype: str  # "fp32" | "bf16"

    @property
    def shape(self):
        return self.data.shape

    def f32(self, index=Ellipsis) -> np.ndarray:
        """The exact values (as float32) of a slice."""
        x = self.data[index]
        return bf16_to_f32(x) if self.dtype == "bf16" else np.asarray(x, dtype=np.float32)

    def f64(self, index=Ellipsis) -> np.ndarray:
        return self.f32(index).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor(bf16_bits(x32), "bf16")
    if dtype == "fp32":
        return Tensor(np.ascontiguousarray(x32, dtype=np.float32), "fp32")
    raise ValueError(dtype)


def _ar1_rows(eps: np.ndarray, rho: float, init: np.ndarray | None = None) -> np.ndarray:
    """AR(1) along axis 0 of eps ([T, d], float64). init is k_{-1} (None: k_0 = e_0)."""
    from scipy.signal import lfilter

    c = math.sqrt(1.0 - rho * rho)
    x = np.empty_like(eps)
    if init is None:
        x[0] = eps[0]
        if eps.shape[0] > 1:
            x[1:] = lfilter([c], [1.0, -rho], eps[1:], axis=0, zi=(rho * eps[0])[None, :])[0]
    else:
        x[:] = lfilter([c], [1.0, -rho], eps, axis=0, zi=(rho * init)[None, :])[0]
    return x


@dataclasses.dataclass
class Prefill:
    q: Tensor
    k: Tensor
    v: Tensor
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    C: int
    K: int
    g: int
    dtype: str
    # Planted-needle bookkeeping (long-prefill workload only): per (b, r) the needle leaves,
    # per (b, h) the needle query positions.
    needle_leaves: np.ndarray | None = None
    needle_queries: np.ndarray | None = None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def make_prefill(*, B: int, Hq: int, Hkv: int, N: int, d: int, C: int, K: int, g: int = 2,
                 dtype: str = "bf16", keys: str = "ar1", rho: float = 0.9, needles: bool = False,
                 n_needle_leaves: int = 8, needle_query_frac: float = 0.01, seed: int = 0,
                 workload_id: int = 0) -> Prefill:
    """Seeded prefill inputs (see module docstring for the recipe)."""
    assert Hq % Hkv == 0
    rq = rng_for(seed, workload_id, STREAM_Q)
    rk = rng_for(seed, workload_id, STREAM_K)
    rv = rng_for(seed, workload_id, STREAM_V)
    q32 = rq.standard_normal((B, Hq, N, d), dtype=np.float32)
    v32 = rv.standard_normal((B, Hkv, N, d), dtype=np.float32)
    k32 = np.empty((B, Hkv, N, d), dtype=np.float32)
    for b in range(B):
        for r in range(Hkv):
            eps = rk.standard_normal((N, d), dtype=np.float32)
            if keys == "ar1":
                k32[b, r] = _ar1_rows(eps.astype(np.float64), rho).astype(np.float32)
            elif keys == "iid":
                k32[b, r] = eps
            else:
                raise ValueError(keys)
    needle_leaves = needle_queries = None
    if needles:
        n0 = -(-N // C)
        G = Hq // Hkv
        rd = rng_for(seed, workload_id, STREAM_NEEDLE_DIR)
        rl = rng_for(seed, workload_id, STREAM_NEEDLE_LEAVES)
        rqn = rng_for(seed, workload_id, STREAM_NEEDLE_QUERIES)
        u = np.empty((B, Hkv, d), dtype=np.float64)
        for b in range(B):
            for r in range(Hkv):
                z = rd.standard_normal(d)
                u[b, r] = z / np.linalg.norm(z)
        nl = min(n_needle_leaves, n0)
        needle_leaves = np.empty((B, Hkv, nl), dtype=np.int64)
        for b in range(B):
            for r in range(Hkv):
                leaves = np.sort(rl.choice(n0, size=nl, replace=False))
                needle_leaves[b, r] = leaves
                for j in leaves:
                    t0, t1 = j * C, min(N, (j + 1) * C)
                    noise = rl.standard_normal((t1 - t0, d)) * 0.5
                    k32[b, r, t0:t1] = (4.0 * u[b, r][None, :] + noise).astype(np.float32)
        nq = int(math.floor(needle_query_frac * N))
        needle_queries = np.empty((B, Hq, nq), dtype=np.int64)
        for b in range(B):
            for h in range(Hq):
                pos = np.sort(rqn.choice(N, size=nq, replace=False))
                needle_queries[b, h] = pos
                noise = rqn.standard_normal((nq, d))
                q32[b, h, pos] = (3.0 * u[b, h // G][None, :] + noise).astype(np.float32)
    return Prefill(q=_store(q32, dtype), k=_store(k32, dtype), v=_store(v32, dtype), B=B, Hq=Hq, Hkv=Hkv,
                   N=N, d=d, C=C, K=K, g=g, dtype=dtype, needle_leaves=needle_leaves,
                   needle_queries=needle_queries)


@dataclasses.dataclass
class Decode:
    """A prefilled cache of `N0` tokens per sequence plus `steps` new tokens per sequence."""

    k_cache: Tensor  # [B, Hkv, Nmax, d]; tokens >= N0 are zero until the steps fill them
    v_cache: Tensor
    q_new: Tensor  # [steps, B, Hq, d]
    k_new: Tensor  # [steps, B, Hkv, d]
    v_new: Tensor
    lens0: np.ndarray  # [B] tokens cached before step 0
    B: int
    Hq: int
    Hkv: int
    Nmax: int
    d: int
    C: int
    K: int
    g: int
    steps: int
    dtype: str

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def make_decode(*, B: int, Hq: int, Hkv: int, N0, d: int, C: int, K: int, steps: int, Nmax: int | None = None,
                g: int = 2, dtype: str = "bf16", rho: float = 0.9, seed: int = 0, workload_id: int = 0) -> Decode:
    """Seeded decode inputs: an AR(1)-key cache of N0 tokens (an int, or one length per sequence) and
    `steps` new tokens per sequence whose keys continue each (b, r) AR(1) chain."""
    lens0 = np.broadcast_to(np.asarray(N0, dtype=np.int64), (B,)).copy()
    Nmax = int(Nmax if Nmax is not None else lens0.max() + steps)
    assert Nmax >= lens0.max() + steps
    rk = rng_for(seed, workload_id, STREAM_K)
    rv = rng_for(seed, workload_id, STREAM_V)
    rdq = rng_for(seed, workload_id, STREAM_DEC_Q)
    rdk = rng_for(seed, workload_id, STREAM_DEC_K)
    rdv = rng_for(seed, workload_id, STREAM_DEC_V)
    store_k = np.zeros((B, Hkv, Nmax, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    store_v = np.zeros_like(store_k)
    k_new32 = np.empty((steps, B, Hkv, d), dtype=np.float32)
    eps_new = rdk.standard_normal((steps, B, Hkv, d), dtype=np.float32).astype(np.float64)
    for b in range(B):
        n0 = int(lens0[b])
        for r in range(Hkv):
            eps = rk.standard_normal((n0, d), dtype=np.float32).astype(np.float64)
            kk = _ar1_rows(eps, rho)
            tail = _ar1_rows(eps_new[:, b, r, :], rho, init=kk[-1])
            k_new32[:, b, r] = tail.astype(np.float32)
            vv = rv.standard_normal((n0, d), dtype=np.float32)
            store_k[b, r, :n0] = _store(kk.astype(np.float32), dtype).data
            store_v[b, r, :n0] = _store(vv, dtype).data
    q_new32 = rdq.standard_normal((steps, B, Hq, d), dtype=np.float32)
    v_new32 = rdv.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    return Decode(k_cache=Tensor(store_k, dtype), v_cache=Tensor(store_v, dtype), q_new=_store(q_new32, dtype),
                  k_new=_store(k_new32, dtype), v_new=_store(v_new32, dtype), lens0=lens0, B=B, Hq=Hq, Hkv=Hkv,
                  Nmax=Nmax, d=d, C=C, K=K, g=g, steps=steps, dtype=dtype)


# Named workloads (the pages' sizes). Each is (builder, kwargs).
WORKLOADS = {
    # tiny fp32 prefill: i.i.d. Q,K,V; 32 leaves of 32 tokens
    "prefill_1k_fp32": dict(kind="prefill", B=1, Hq=1, Hkv=1, N=1024, d=64, C=32, K=4, dtype="fp32", keys="iid",
                            workload_id=1),
    # 16K-token GQA prefill (8 query heads per KV head)
    "prefill_16k": dict(kind="prefill", B=1, Hq=16, Hkv=2, N=16384, d=128, C=64, K=16, dtype="bf16", keys="ar1",
                        workload_id=2),
    # 64K-token GQA prefill (4 query heads per KV head)
    "prefill_64k": dict(kind="prefill", B=1, Hq=32, Hkv=8, N=65536, d=128, C=64, K=16, dtype="bf16", keys="ar1",
                        workload_id=3),
    # 256K-token GQA prefill with planted needles
    "prefill_256k_needles": dict(kind="prefill", B=1, Hq=32, Hkv=8, N=262144, d=128, C=64, K=16, dtype="bf16",
                                 keys="ar1", needles=True, workload_id=4),
    # decode: 8 sequences with 131072 cached tokens, 256 steps
    "decode_128k": dict(kind="decode", B=8, Hq=32, Hkv=8, N0=131072, Nmax=131328, steps=256, d=128, C=64, K=16,
                        dtype="bf16", workload_id=5),
}


def make_workload(name: str, seed: int = 0, **overrides):
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "prefill":
        return make_prefill(seed=seed, **spec)
    return make_decode(seed=seed, **spec)
