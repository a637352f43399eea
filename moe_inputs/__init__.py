"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, and it is the one piece of code that
both the CPU oracle (through the tests) and the GPU path are fed from.

Recipe (every tensor gets a stream of its own, so any single expert can be
regenerated without drawing the others):

* stream = PCG64(SeedSequence([seed, tensor_id, expert_id]))
  tensor ids: u = 0, E_gate = 1, routed expert = 2, shared expert = 3,
  bias permutation = 4.
* u ~ N(0, 1); gate vectors e_i and every FFN weight ~ N(0, sigma^2), drawn as
  float32 standard normals times sigma.
* bf16 workloads round each float32 draw to bfloat16, round-to-nearest-even.
  The oracle reads those same rounded values (decoded exactly to float32), so
  both sides see identical numbers.
* skewed workloads add a per-expert logit bias b_i = -s * ln(r_i), where r is
  1 + a seeded permutation of 0..N-1; softmax(b) alone is then the Zipf(s)
  profile over the experts.

Weight block layout of one expert (the layout the C ABI takes), row-major,
contiguous:  W_gate [I][d], then W_up [I][d], then W_down [d][I].
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_U, TENSOR_E, TENSOR_ROUTED, TENSOR_SHARED, TENSOR_BIASPERM, TENSOR_DH = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    d: int          # hidden size
    N: int          # routed experts (rows of E_gate)
    K: int          # routed experts kept per token
    K_s: int        # shared experts, always active
    I: int          # SwiGLU intermediate size of one expert
    dtype: str      # "f32" or "bf16": storage type of u, E_gate, weights, h
    sigma: float    # std of gate vectors and FFN weights
    seed: int
    zipf_s: float | None = None   # per-expert logit bias exponent, or None

    def flops_per_token(self) -> int:
        """Algorithmic FLOPs per token: router 2dN + SwiGLU experts 6dI(K+K_s)."""
        return 2 * self.d * self.N + 6 * self.d * self.I * (self.K + self.K_s)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is exercised on.  Shapes follow the paper's
# 2B / 16B / 145B model families (expert counts written as routed + shared).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", T=256, d=256, N=16, K=4, K_s=1, I=128,
                 dtype="f32", sigma=0.02, seed=101),
        Workload("moe2b_bf16", T=4096, d=1280, N=63, K=7, K_s=1, I=896,
                 dtype="bf16", sigma=0.02, seed=102),
        Workload("moe16b_prefill_bf16", T=8192, d=2048, N=64, K=6, K_s=2, I=1408,
                 dtype="bf16", sigma=0.02, seed=103),
        Workload("moe16b_decode_bf16", T=64, d=2048, N=64, K=6, K_s=2, I=1408,
                 dtype="bf16", sigma=0.02, seed=104),
        Workload("moe145b_skewed_bf16", T=16384, d=4096, N=128, K=12, K_s=4, I=1536,
                 dtype="bf16", sigma=0.015, seed=105, zipf_s=1.1),
    ]
}


def _stream(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, expert])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # NaN never occurs in these draws; finite values round by the usual bias trick.
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(seed: int, tensor: int, expert: int, n: int, scale: float, dtype: str):
    """n normal draws times scale, in storage form: float32 array, or uint16 bf16 bits."""
    x = _stream(seed, tensor, expert).standard_normal(n, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


class MoEInputs:
    """Lazily generated inputs of one workload.

    ``*_raw`` accessors return the storage form (float32, or uint16 bf16 bits)
    in the ABI layout; ``*_f32`` accessors return the same values as float32.
    """

    def __init__(self, w: Workload):
        self.w = w
        self._cache: dict = {}

    # -- storage form -------------------------------------------------------
    def u_raw(self) -> np.ndarray:
        w = self.w
        if "u" not in self._cache:
            self._cache["u"] = _draw(w.seed, TENSOR_U, 0, w.T * w.d, 1.0, w.dtype).reshape(w.T, w.d)
        return self._cache["u"]

    def E_gate_raw(self) -> np.ndarray:
        w = self.w
        if "E" not in self._cache:
            self._cache["E"] = _draw(w.seed, TENSOR_E, 0, w.N * w.d, w.sigma, w.dtype).reshape(w.N, w.d)
        return self._cache["E"]

    def routed_block_raw(self, e: int) -> np.ndarray:
        w = self.w
        return _draw(w.seed, TENSOR_ROUTED, e, 3 * w.I * w.d, w.sigma, w.dtype)

    def shared_block_raw(self, j: int) -> np.ndarray:
        w = self.w
        return _draw(w.seed, TENSOR_SHARED, j, 3 * w.I * w.d, w.sigma, w.dtype)

    def routed_all_raw(self, threads: int = 8) -> np.ndarray:
        """All N routed blocks, [N][3*I*d], drawn in parallel (streams are independent)."""
        w = self.w
        out = np.empty((w.N, 3 * w.I * w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)

        def fill(e):
            out[e] = self.routed_block_raw(e)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(w.N)))
        return out

    def shared_all_raw(self) -> np.ndarray:
        w = self.w
        out = np.empty((w.K_s, 3 * w.I * w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        for j in range(w.K_s):
            out[j] = self.shared_block_raw(j)
        return out

    def dh_raw(self) -> np.ndarray:
        """Upstream gradient of the layer output for the backward pass, [T][d], N(0, 1)."""
        w = self.w
        if "dh" not in self._cache:
            self._cache["dh"] = _draw(w.seed, TENSOR_DH, 0, w.T * w.d, 1.0, w.dtype).reshape(w.T, w.d)
        return self._cache["dh"]

    def gate_bias(self) -> np.ndarray | None:
        """Per-expert logit bias (float32) for skewed workloads, else None."""
        w = self.w
        if w.zipf_s is None:
            return None
        r = 1 + _stream(w.seed, TENSOR_BIASPERM, 0).permutation(w.N)
        return (-w.zipf_s * np.log(r.astype(np.float64))).astype(np.float32)

    # -- float32 views for the oracle --------------------------------------
    def _to_f32(self, raw: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(raw) if self.w.dtype == "bf16" else raw

    def u_f32(self) -> np.ndarray:
        return self._to_f32(self.u_raw())

    def E_gate_f32(self) -> np.ndarray:
        return self._to_f32(self.E_gate_raw())

    def dh_f32(self) -> np.ndarray:
        return self._to_f32(self.dh_raw())

    def split_block(self, block: np.ndarray):
        """(W_gate [I][d], W_up [I][d], W_down [d][I]) views of one expert block."""
        w = self.w
        Id = w.I * w.d
        return (block[:Id].reshape(w.I, w.d), block[Id:2 * Id].reshape(w.I, w.d),
                block[2 * Id:].reshape(w.d, w.I))

    def routed_expert_f32(self, e: int):
        return self.split_block(self._to_f32(self.routed_block_raw(e)))

    def shared_expert_f32(self, j: int):
        return self.split_block(self._to_f32(self.shared_block_raw(j)))


def make(name_or_workload, **overrides) -> MoEInputs:
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    if overrides:
        w = w.replace(**overrides)
    return MoEInputs(w)


def custom(T, d, N, K, K_s, I, dtype="f32", sigma=0.02, seed=7, zipf_s=None, name="custom") -> MoEInputs:
    return MoEInputs(Workload(name, T, d, N, K, K_s, I, dtype, sigma, seed, zipf_s))


__all__ = ["Workload", "WORKLOADS", "MoEInputs", "make", "custom",
           "f32_to_bf16_bits", "bf16_bits_to_f32"]


# Granularity sweep at equal parameters and equal compute (DeepSeekMoE paper
# summary, papercache.org, sec. 3.1 fine-grained expert segmentation and
# sec. 3.2 shared expert isolation, Fig. 2): a conventional layer of N0
# experts of intermediate size I0 with top-K0 routing is cut into m * N0
# experts of size I0 / m with top m * K0; K_s of those experts then become
# shared, leaving m * N0 - K_s routed experts with top m * K0 - K_s.  m = 1,
# K_s = 0 is the conventional top-2 layer.
GRANULARITY_SWEEP = [(1, 0), (1, 1), (2, 0), (2, 1), (4, 0), (4, 1), (8, 0), (8, 1)]


def granularity(m: int, K_s: int, T: int = 8192, d: int = 2048, N0: int = 16, K0: int = 2,
                I0: int = 5632, dtype: str = "bf16", sigma: float = 0.02, seed: int = 110) -> Workload:
    if I0 % m != 0:
        raise ValueError("I0 must split into m equal parts")
    return Workload(f"gran_m{m}_ks{K_s}", T=T, d=d, N=m * N0 - K_s, K=m * K0 - K_s, K_s=K_s,
                    I=I0 // m, dtype=dtype, sigma=sigma, seed=seed + 10 * m + K_s)
