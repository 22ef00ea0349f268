"""Seeded synthetic workloads shaped like the pages' benchmarks.

This module only draws random numbers and names shapes; it holds none of the
quantization or attention arithmetic.  Both the GPU tests/benchmark and the
CPU oracle take their inputs from here.

Recipe: ``rng = numpy.random.default_rng(seed)``; every tensor is drawn as
float32 (uniform [0, 1) or standard normal) in the order q, K, V (then, for
the append workload, k_new, v_new, q per step) and cast round-to-nearest-even
to its storage dtype.  Storage conventions: "f32" -> np.float32,
"f16" -> np.float16, "bf16" -> np.uint16 bit patterns.

Shapes follow the MLX benchmark on the page "add fast::quantized_kv_update"
(sdpa_vector_bench.py: B=1, H=32, H_k=8, D=128, L=65536, uniform inputs,
4-bit, group 64) and the llama.cpp page "Metal: Optimize q8_0 KV - #25556"
(GQA-16, head size 256, decode at 20K depth, 512-query prompts at 20K).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hk: int
    D: int
    L: int                 # attended length (decode / prefill); initial length for append
    Lq: int
    dtype: str             # q / K / V storage dtype
    dist: str              # "uniform" or "normal"
    mode: str              # "affine" or "q8_0"
    bits: int
    group_size: int
    scale: float
    causal: bool
    seed: int
    steps: int = 0         # append+decode steps (append workload only)
    L_cap: int = 0         # cache capacity (0 -> L)

    @property
    def cap(self) -> int:
        return self.L_cap or self.L

    @property
    def G(self) -> int:
        return self.Hq // self.Hk


WORKLOADS = {
    "tiny_decode": Workload("tiny_decode", 1, 4, 1, 64, 256, 1, "f32", "uniform", "affine", 8, 64,
                            1.0, False, 101),
    "decode_64k_4bit_gqa4": Workload("decode_64k_4bit_gqa4", 1, 32, 8, 128, 65536, 1, "f16",
                                     "uniform", "affine", 4, 64, 1.0, False, 3),
    "append_decode_b8_8bit": Workload("append_decode_b8_8bit", 8, 32, 8, 128, 16384, 1, "f16",
                                      "normal", "affine", 8, 64, 1.0 / math.sqrt(128.0), False,
                                      303, steps=64, L_cap=16448),
    "q8_0_decode_gqa16": Workload("q8_0_decode_gqa16", 1, 32, 2, 256, 20480, 1, "f16", "normal",
                                  "q8_0", 8, 32, 1.0 / 16.0, False, 404),
    "q8_0_prefill_512": Workload("q8_0_prefill_512", 1, 32, 2, 256, 20480, 512, "f16", "normal",
                                 "q8_0", 8, 32, 1.0 / 16.0, True, 505),
    # the wider formats at the 64K GQA-4 decode shape (and head size 96 at a
    # 16K context): affine 3-bit (8 codes in 3 bytes), the symmetric 4-bit
    # blocks (the Q4_0 reading), affine 4-bit group 32 at D = 96
    "decode_64k_3bit_gqa4": Workload("decode_64k_3bit_gqa4", 1, 32, 8, 128, 65536, 1, "f16",
                                     "uniform", "affine", 3, 64, 1.0, False, 3),
    "decode_64k_qsym4_gqa4": Workload("decode_64k_qsym4_gqa4", 1, 32, 8, 128, 65536, 1, "f16",
                                      "normal", "qsym", 4, 32, 1.0 / math.sqrt(128.0), False, 7),
    "decode_16k_d96_gqa4": Workload("decode_16k_d96_gqa4", 1, 32, 8, 96, 16384, 1, "f16", "normal",
                                    "affine", 4, 32, 1.0 / math.sqrt(96.0), False, 9),
    # the unquantized baseline at the shapes of the two decode workloads: dense
    # fp16 K/V (the sdpa baseline of the MLX benchmark; the F16 cache of the
    # llama.cpp page), same distributions as the quantized workloads
    "dense_decode_64k_gqa4": Workload("dense_decode_64k_gqa4", 1, 32, 8, 128, 65536, 1, "f16",
                                      "uniform", "dense", 16, 128, 1.0, False, 3),
    "dense_decode_20k_gqa16": Workload("dense_decode_20k_gqa16", 1, 32, 2, 256, 20480, 1, "f16",
                                       "normal", "dense", 16, 256, 1.0 / 16.0, False, 404),
}


def cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round-to-nearest-even cast of float32 draws to a storage dtype."""
    if dtype == "f32":
        return x32.astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def draw(rng: np.random.Generator, shape, dist: str, dtype: str) -> np.ndarray:
    if dist == "uniform":
        x = rng.random(shape, dtype=np.float32)
    elif dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError(dist)
    return cast(x, dtype)


def make_inputs(w: Workload, L: int | None = None, Lq: int | None = None,
                B: int | None = None) -> dict:
    """q [B,Hq,Lq,D], k, v [B,Hk,L,D] for a workload (sizes may be overridden
    to shrink a case while keeping its distribution and structure)."""
    L = w.L if L is None else L
    Lq = w.Lq if Lq is None else Lq
    B = w.B if B is None else B
    rng = np.random.default_rng(w.seed)
    q = draw(rng, (B, w.Hq, Lq, w.D), w.dist, w.dtype)
    k = draw(rng, (B, w.Hk, L, w.D), w.dist, w.dtype)
    v = draw(rng, (B, w.Hk, L, w.D), w.dist, w.dtype)
    return {"q": q, "k": k, "v": v, "rng": rng}


def append_step_inputs(w: Workload, rng: np.random.Generator, B: int | None = None) -> dict:
    """One append+decode step: k_new, v_new [B,Hk,1,D], q [B,Hq,1,D]."""
    B = w.B if B is None else B
    k_new = draw(rng, (B, w.Hk, 1, w.D), w.dist, w.dtype)
    v_new = draw(rng, (B, w.Hk, 1, w.D), w.dist, w.dtype)
    q = draw(rng, (B, w.Hq, 1, w.D), w.dist, w.dtype)
    return {"k_new": k_new, "v_new": v_new, "q": q}


def random_case(seed: int, shape, dist: str = "normal", dtype: str = "f16") -> np.ndarray:
    """A seeded tensor for small fuzz cases."""
    return draw(np.random.default_rng(seed), shape, dist, dtype)


def to_tensor(a: np.ndarray, dtype: str, device="cuda"):
    """A storage array (see the module docstring) as a torch tensor on device."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)
