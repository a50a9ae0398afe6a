"""Seeded synthetic workloads for the weight-only block-32 matmul.

This module holds only workload shapes and random-number recipes; it contains
none of the method's arithmetic (no quantization, no matmul), so both the HIP
path and the CPU oracle can draw the same inputs from it.

Shapes follow the Qwen3-0.6B-style decoder of MOSS-Transcribe-Diarize: hidden
size 1024 (the moss-transcribe-diarize-litert card, "Files": audio embeds
(1,375,1024)), 28 layers with 8 KV heads of 128 (same table, the decoder's
external KV cache 28x2 x (1,N,8,128)); the q width 2048, the MLP width 3072 and
the vocabulary 151936 are the standard Qwen3-0.6B sizes. Token counts: M=1 is
the card's ``decode`` signature, M=128 and M=1024 its ``prefill_128`` and
``prefill_1024`` signatures, M=4096 about 5.5 minutes of audio at the 12.5
audio tokens per second of the soniqo guide ("Limits and memory").

Random recipe: numpy ``Generator(PCG64(seed))``, ``standard_normal`` drawn
directly in float32, multiplied by the float32 standard deviation (0.02 for
weights, 1 for activations). The single-GEMV workload draws W then x from
PCG64(0). Every other weight tensor is seeded by ``SeedSequence([config, layer,
proj, 0])`` (the same model at every M) and every activation by
``SeedSequence([config, M, layer, proj, role])``, with proj q0 k1 v2 o3 gate4
up5 down6 lm_head7 and role 1 activation, 2 outlier-row choice. Config ids:
0 single GEMV, 1 decode step, 2 layer prefill, 3 mixed decode, 4 long prefill.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

HIDDEN = 1024
Q_DIM = 2048
KV_DIM = 1024
INTER = 3072
VOCAB = 151936
LAYERS = 28
BLOCK = 32

W_SIGMA = 0.02
X_SIGMA = 1.0

PROJ_ID = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "lm_head": 7}

# (name, K, N, activation group). Projections that read the same tensor in a
# real layer share one synthetic activation: q/k/v the attention input, gate/up
# the MLP input; o and down read their own.
LAYER_PROJS: List[Tuple[str, int, int, str]] = [
    ("q", HIDDEN, Q_DIM, "attn"),
    ("k", HIDDEN, KV_DIM, "attn"),
    ("v", HIDDEN, KV_DIM, "attn"),
    ("o", Q_DIM, HIDDEN, "o"),
    ("gate", HIDDEN, INTER, "mlp"),
    ("up", HIDDEN, INTER, "mlp"),
    ("down", INTER, HIDDEN, "down"),
]
PROJ_N = {name: N for name, _, N, _ in LAYER_PROJS}
# Shared-input fusion: projections that read the same activation, stacked along
# N into one tensor (q|k|v 1024->4096, gate|up 1024->6144).
FUSED_PROJS: List[Tuple[str, Tuple[str, ...]]] = [("qkv", ("q", "k", "v")), ("o", ("o",)),
                                                 ("gateup", ("gate", "up")), ("down", ("down",))]
# activation group -> projection whose id seeds it
_GROUP_SEED_PROJ = {"attn": "q", "o": "o", "mlp": "gate", "down": "down", "lm": "lm_head"}


@dataclass(frozen=True)
class TensorSpec:
    name: str          # e.g. "L3.gate" or "lm_head"
    layer: int
    proj: str
    K: int
    N: int
    bits: int
    act: str           # key of the activation it reads
    act_row0: int = 0  # first activation row it reads (for row-offset views)
    M: int = 0         # rows it reads
    parts: Tuple[str, ...] = ()   # fused tensor: projections whose rows are stacked along N

    @property
    def q_bytes(self) -> int:
        return self.N * self.K * self.bits // 8

    @property
    def s_bytes(self) -> int:
        return self.N * (self.K // BLOCK) * 2

    @property
    def weight_bytes(self) -> int:
        return self.q_bytes + self.s_bytes


@dataclass(frozen=True)
class ActSpec:
    key: str
    M: int
    K: int
    seed: Tuple[int, ...]
    outlier_rows: int = 0          # rows scaled by OUTLIER_GAIN
    outlier_seed: Tuple[int, ...] = ()


OUTLIER_GAIN = np.float32(20.0)


@dataclass
class Workload:
    name: str
    config: int
    M: int
    tensors: List[TensorSpec]
    acts: Dict[str, ActSpec]
    description: str = ""
    # single-stream recipe (the single-GEMV workload draws W then x from one seed)
    single_stream_seed: Optional[int] = None
    _cache: Dict[str, np.ndarray] = field(default_factory=dict, repr=False)

    # ---- sizes ----
    @property
    def weight_bytes(self) -> int:
        return sum(t.weight_bytes for t in self.tensors)

    @property
    def flops(self) -> int:
        return sum(2 * t.M * t.N * t.K for t in self.tensors)

    @property
    def act_bytes(self) -> int:
        """x bytes, each call reading its own x once (shared inputs count per call)."""
        return sum(4 * t.M * t.K for t in self.tensors)

    @property
    def out_bytes(self) -> int:
        return sum(4 * t.M * t.N for t in self.tensors)

    @property
    def total_bytes(self) -> int:
        """Algorithmic HBM bytes: packed weights + scales, each call's x read once, y written once."""
        return self.weight_bytes + self.act_bytes + self.out_bytes

    # ---- draws ----
    def weight(self, t: TensorSpec) -> np.ndarray:
        """fp32 [N, K] weights of tensor t."""
        if self.single_stream_seed is not None:
            w, _ = self._single_stream()
            return w
        if t.parts:
            # a fused tensor is its projections' own weights, stacked along N
            return np.concatenate([self._draw(t.layer, p, PROJ_N[p], t.K) for p in t.parts], axis=0)
        return self._draw(t.layer, t.proj, t.N, t.K)

    def _draw(self, layer: int, proj: str, N: int, K: int) -> np.ndarray:
        ss = np.random.SeedSequence([self.config, layer, PROJ_ID[proj], 0])
        rng = np.random.Generator(np.random.PCG64(ss))
        w = rng.standard_normal((N, K), dtype=np.float32)
        w *= np.float32(W_SIGMA)
        return w

    def activation(self, key: str) -> np.ndarray:
        """fp32 [M, K] activation `key` (cached: activations are small)."""
        if key in self._cache:
            return self._cache[key]
        a = self.acts[key]
        if self.single_stream_seed is not None:
            _, x = self._single_stream()
        else:
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(a.seed))))
            x = rng.standard_normal((a.M, a.K), dtype=np.float32)
            if X_SIGMA != 1.0:
                x *= np.float32(X_SIGMA)
            if a.outlier_rows:
                prng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(a.outlier_seed))))
                rows = prng.permutation(a.M)[: a.outlier_rows]
                x[np.sort(rows)] *= OUTLIER_GAIN
        self._cache[key] = x
        return x

    def x_for(self, t: TensorSpec) -> np.ndarray:
        x = self.activation(t.act)
        return x[t.act_row0: t.act_row0 + t.M]

    def _single_stream(self):
        if "__w" not in self._cache:
            t = self.tensors[0]
            rng = np.random.Generator(np.random.PCG64(self.single_stream_seed))
            w = rng.standard_normal((t.N, t.K), dtype=np.float32)
            w *= np.float32(W_SIGMA)
            x = rng.standard_normal((t.M, t.K), dtype=np.float32)
            self._cache["__w"] = w
            self._cache["__x"] = x
        return self._cache["__w"], self._cache["__x"]


def _act(config: int, M: int, layer: int, group: str, K: int, outliers: bool = False) -> ActSpec:
    pid = PROJ_ID[_GROUP_SEED_PROJ[group]]
    n_out = max(1, int(round(0.01 * M))) if outliers else 0
    return ActSpec(key=f"L{layer}.{group}" if group != "lm" else "lm", M=M, K=K,
                   seed=(config, M, layer, pid, 1), outlier_rows=n_out,
                   outlier_seed=(config, M, layer, pid, 2))


def single_gemv() -> Workload:
    """Single int4 block-32 GEMV, M=1, K=1024, N=2048 (the q-projection shape), seed 0."""
    t = TensorSpec("q", 0, "q", HIDDEN, Q_DIM, 4, act="x", M=1)
    acts = {"x": ActSpec("x", 1, HIDDEN, seed=(0,))}
    return Workload("single_gemv_int4_m1_k1024_n2048", 0, 1, [t], acts,
                    description="one int4 GEMV, M=1, 1024->2048", single_stream_seed=0)


def decode_step(M: int = 1, mixed: bool = False, fused: bool = False, proj_bits: int = 4) -> Workload:
    """One decode step: 28 layers x 7 projections + the tied lm_head (int8).

    int4 everywhere but the lm_head; with ``mixed`` the attention projections
    (q, k, v, o) are int8 and the MLP (gate, up, down) int4. With ``fused`` the
    projections that share an input are stacked along N (q|k|v, gate|up): the
    same weights and activations, 113 GEMVs instead of 197. ``proj_bits`` = 5
    packs every projection in int5 (the MLX default of the soniqo guide), the
    lm_head staying int8.
    """
    config = 3 if mixed else 1
    tensors: List[TensorSpec] = []
    acts: Dict[str, ActSpec] = {}
    proj = {name: (K, group) for name, K, _, group in LAYER_PROJS}
    for layer in range(LAYERS):
        groups = FUSED_PROJS if fused else [(name, (name,)) for name, _, _, _ in LAYER_PROJS]
        for name, parts in groups:
            K, group = proj[parts[0]]
            N = sum(PROJ_N[p] for p in parts)
            bits = 8 if (mixed and group in ("attn", "o")) else proj_bits
            key = f"L{layer}.{group}"
            if key not in acts:
                acts[key] = _act(config, M, layer, group, K)
            tensors.append(TensorSpec(f"L{layer}.{name}", layer, parts[0] if len(parts) == 1 else name, K, N,
                                      bits, act=key, M=M, parts=parts if len(parts) > 1 else ()))
    acts["lm"] = _act(config, M, 0, "lm", HIDDEN)
    tensors.append(TensorSpec("lm_head", 0, "lm_head", HIDDEN, VOCAB, 8, act="lm", M=M))
    kind = "mixed int8-attn/int4-mlp" if mixed else f"int{proj_bits}"
    return Workload(f"decode_step_{'mixed' if mixed else kind}_m{M}{'_fused' if fused else ''}", config, M,
                    tensors, acts,
                    description=f"one decode step, M={M}, {kind}, {len(tensors)} GEMVs incl. int8 lm_head"
                                + (", q|k|v and gate|up stacked along N" if fused else ""))


def prefill_layer(M: int) -> Workload:
    """Prefill through the seven int4 projections of one layer; 1% of x rows scaled x20."""
    config = 2
    tensors: List[TensorSpec] = []
    acts: Dict[str, ActSpec] = {}
    for name, K, N, group in LAYER_PROJS:
        key = f"L0.{group}"
        if key not in acts:
            acts[key] = _act(config, M, 0, group, K, outliers=True)
        tensors.append(TensorSpec(name, 0, name, K, N, 4, act=key, M=M))
    return Workload(f"prefill_layer_int4_m{M}", config, M, tensors, acts,
                    description=f"prefill, M={M}, 7 int4 projections, 1% outlier rows x20")


def long_prefill(M: int = 4096, lm_rows: int = 64) -> Workload:
    """Long-audio prefill: gate/up/down at M=4096 (int4) + int8 lm_head on the last 64 rows."""
    config = 4
    acts = {
        "L0.mlp": _act(config, M, 0, "mlp", HIDDEN),
        "L0.down": _act(config, M, 0, "down", INTER),
    }
    tensors = [
        TensorSpec("gate", 0, "gate", HIDDEN, INTER, 4, act="L0.mlp", M=M),
        TensorSpec("up", 0, "up", HIDDEN, INTER, 4, act="L0.mlp", M=M),
        TensorSpec("down", 0, "down", INTER, HIDDEN, 4, act="L0.down", M=M),
        TensorSpec("lm_head", 0, "lm_head", HIDDEN, VOCAB, 8, act="L0.mlp",
                   act_row0=M - lm_rows, M=lm_rows),
    ]
    return Workload(f"long_prefill_m{M}", config, M, tensors, acts,
                    description=f"gate/up/down int4 at M={M} + int8 lm_head on the last {lm_rows} rows")


def workload(name: str) -> Workload:
    """Named workloads: single_gemv, decode_step, decode_step_fused, prefill_128,
    prefill_1024, mixed_m{1,2,4,8,16}, long_prefill."""
    if name == "single_gemv":
        return single_gemv()
    if name == "decode_step":
        return decode_step(1, mixed=False)
    if name == "decode_step_fused":
        return decode_step(1, mixed=False, fused=True)
    if name.startswith("prefill_"):
        return prefill_layer(int(name.split("_")[1]))
    if name.startswith("mixed_m"):
        return decode_step(int(name[len("mixed_m"):]), mixed=True)
    if name == "long_prefill":
        return long_prefill()
    raise KeyError(name)


ALL_WORKLOADS = ["single_gemv", "decode_step", "prefill_128", "prefill_1024",
                 "mixed_m1", "mixed_m2", "mixed_m4", "mixed_m8", "mixed_m16", "long_prefill"]


def normal(shape, seed, sigma: float = 1.0) -> np.ndarray:
    """Generic seeded fp32 normal draw for tests (seed: int or tuple)."""
    ss = np.random.SeedSequence(list(seed) if isinstance(seed, (tuple, list)) else seed)
    rng = np.random.Generator(np.random.PCG64(ss))
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def generator(seed) -> np.random.Generator:
    ss = np.random.SeedSequence(list(seed) if isinstance(seed, (tuple, list)) else seed)
    return np.random.Generator(np.random.PCG64(ss))
