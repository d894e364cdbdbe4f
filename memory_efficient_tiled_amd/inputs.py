"""Seeded synthetic inputs and the named workloads.

This module is shared by the oracle's tests, the GPU parity tests and the
bench.  It holds none of the attention arithmetic: it draws Gaussian tensors
from a seeded PCG64 stream, rounds them to the 16-bit input type and describes
the workload shapes.  Both sides of every parity check read the same arrays.

Workload shapes follow the pages:
  * the isolated attention sweep (B=1, H=16, D=64, fp16) of the English
    noflash-attention post at ai-navigate-news.com, section "It's actually
    faster too!" (its benchmark table);
  * the GQA decoder shape behind the Qwen 2.5 0.5B table of the same post,
    section "Where it landed" (14 query heads over 2 KV heads, D=64);
  * the 17K- and 75K-token video sequences of the same post, section
    "The problem" (24 heads: the score-matrix sizes quoted there are
    24 x N^2 x 4 bytes).
The pages publish no tensors, so every input is synthetic.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F16 = "f16"
BF16 = "bf16"
FP8 = "fp8"      # OCP E4M3 bytes with one descale factor per tensor


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str
    causal: bool
    k_offset_std: float | None = None   # per-channel offset added to K
    sampled_rows: int | None = None      # oracle rows per head at full size
    note: str = ""
    Dv_: int | None = None               # V/O head dimension when it differs from D

    @property
    def Dv(self) -> int:
        return self.D if self.Dv_ is None else self.Dv_

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Algorithmic flops: 2*B*Hq*Nq*Nkv*(D + Dv) (4*...*D when Dv = D),
        halved when causal."""
        f = 2.0 * self.B * self.Hq * self.Nq * self.Nkv * (self.D + self.Dv)
        return f / 2.0 if self.causal else f

    @property
    def bwd_flops(self) -> float:
        """Algorithmic flops of the gradients: S, dP, dV, dK, dQ, i.e.
        2*B*Hq*Nq*Nkv*(3*D + 2*Dv) (10*...*D when Dv = D, 2.5x the forward),
        halved when causal."""
        f = 2.0 * self.B * self.Hq * self.Nq * self.Nkv * (3 * self.D + 2 * self.Dv)
        return f / 2.0 if self.causal else f

    @property
    def hbm_bytes(self) -> float:
        """Algorithmic HBM bytes of one forward: Q, K, V read once, O written
        once (2 bytes an element; 1 for FP8 inputs), LSE written once (fp32)."""
        e = 1 if self.dtype == FP8 else 2
        q = self.B * self.Hq * self.Nq * self.D
        kv = self.B * self.Hkv * self.Nkv * (self.D + self.Dv)
        o = self.B * self.Hq * self.Nq * self.Dv
        return float(e * (q + kv) + 2 * o + 4 * self.B * self.Hq * self.Nq)

    @property
    def bound(self) -> str:
        """The roofline bound: "hbm" below the MI355X ridge of 2.5e15 / 8e12
        = 312.5 flop per byte, else "mfma"."""
        return "hbm" if self.flops / self.hbm_bytes < 2.5e15 / 8e12 else "mfma"

    def describe(self) -> str:
        dv = f" Dv={self.Dv}" if self.Dv != self.D else ""
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} Nq={self.Nq} "
                f"Nkv={self.Nkv} D={self.D}{dv} {self.dtype} "
                f"{'causal' if self.causal else 'non-causal'}")


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS: dict[str, Workload] = {}
WORKLOADS["tiny-256"] = _w(name="tiny-256", B=1, Hq=16, Hkv=16, Nq=256, Nkv=256,
                           D=64, dtype=F16, causal=False,
                           note="tiny non-causal MHA")
for _n in (1024, 2048, 4096, 8192, 16384):
    WORKLOADS[f"sweep-{_n}"] = _w(name=f"sweep-{_n}", B=1, Hq=16, Hkv=16, Nq=_n,
                                  Nkv=_n, D=64, dtype=F16, causal=False,
                                  note="isolated MHA sweep")
for _n in (4096, 8192, 16384):
    WORKLOADS[f"gqa-causal-{_n}"] = _w(name=f"gqa-causal-{_n}", B=1, Hq=14, Hkv=2,
                                       Nq=_n, Nkv=_n, D=64, dtype=F16, causal=True,
                                       note="causal GQA decoder prefill")
WORKLOADS["dit-17160"] = _w(name="dit-17160", B=1, Hq=24, Hkv=24, Nq=17160,
                            Nkv=17160, D=128, dtype=BF16, causal=False,
                            k_offset_std=0.5,
                            note="video-DiT self-attention, K per-channel offset")
WORKLOADS["dit-75600"] = _w(name="dit-75600", B=1, Hq=24, Hkv=24, Nq=75600,
                            Nkv=75600, D=128, dtype=BF16, causal=False,
                            sampled_rows=256,
                            note="long video-DiT self-attention")

# Decode: one new query row per head over a 64K-token cache, 16 query heads
# on 2 KV heads (the GQA grouping the post flattens, section "The DIY
# approach"; its long-context LLM table, section "Where it landed").  HBM-
# bound: K and V are read once per KV head when the 8 query heads of a group
# are packed into one tile.
WORKLOADS["decode-64k"] = _w(name="decode-64k", B=1, Hq=16, Hkv=2, Nq=1, Nkv=65536,
                             D=128, dtype=BF16, causal=False,
                             note="GQA decode over a 64K-token cache")

# Head dimension 256, beyond the pages' 64/128 (the scope's list of further
# head dimensions): an MHA sweep point and a causal GQA prefill shape.
WORKLOADS["hd256-8192"] = _w(name="hd256-8192", B=1, Hq=16, Hkv=16, Nq=8192, Nkv=8192,
                             D=256, dtype=BF16, causal=False,
                             note="head dim 256, non-causal MHA")
WORKLOADS["hd256-gqa-causal-8192"] = _w(name="hd256-gqa-causal-8192", B=1, Hq=16, Hkv=8,
                                        Nq=8192, Nkv=8192, D=256, dtype=BF16, causal=True,
                                        note="head dim 256, causal GQA prefill")

# Head dimension 96 (same list): MHA, non-causal and causal, 8192 tokens.
WORKLOADS["hd96-8192"] = _w(name="hd96-8192", B=1, Hq=32, Hkv=32, Nq=8192, Nkv=8192,
                            D=96, dtype=BF16, causal=False,
                            note="head dim 96, non-causal MHA")
WORKLOADS["hd96-causal-8192"] = _w(name="hd96-causal-8192", B=1, Hq=32, Hkv=32, Nq=8192,
                                   Nkv=8192, D=96, dtype=BF16, causal=True,
                                   note="head dim 96, causal MHA prefill")

# Head dimension 80 (same list): MHA, non-causal, 8192 tokens, fp16.
WORKLOADS["hd80-8192"] = _w(name="hd80-8192", B=1, Hq=32, Hkv=32, Nq=8192, Nkv=8192,
                            D=80, dtype=F16, causal=False,
                            note="head dim 80, non-causal MHA")

# Query/key head dimension 192 with value head dimension 128 (same list:
# Dv != D), the per-head shape of multi-head latent attention at prefill;
# 16 heads, 8192 tokens, causal and not.
WORKLOADS["hd192v128-causal-8192"] = _w(name="hd192v128-causal-8192", B=1, Hq=16, Hkv=16,
                                        Nq=8192, Nkv=8192, D=192, Dv_=128, dtype=BF16,
                                        causal=True, note="head dims 192/128, causal prefill")
WORKLOADS["hd192v128-8192"] = _w(name="hd192v128-8192", B=1, Hq=16, Hkv=16, Nq=8192,
                                 Nkv=8192, D=192, Dv_=128, dtype=BF16, causal=False,
                                 note="head dims 192/128, non-causal")

# 8-bit inputs (no page names a format): the headline shape, and a causal
# GQA prefill at D = 128, both quantised per tensor to E4M3.
WORKLOADS["dit-17160-fp8"] = _w(name="dit-17160-fp8", B=1, Hq=24, Hkv=24, Nq=17160,
                                Nkv=17160, D=128, dtype=FP8, causal=False, k_offset_std=0.5,
                                note="video-DiT self-attention on E4M3 inputs")
WORKLOADS["gqa-causal-fp8-8192"] = _w(name="gqa-causal-fp8-8192", B=1, Hq=32, Hkv=8, Nq=8192,
                                      Nkv=8192, D=128, dtype=FP8, causal=True,
                                      note="causal GQA prefill on E4M3 inputs")

HEADLINE = "dit-17160"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); raw bits.

    Inputs here are finite Gaussian draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def quantize_fp8(x: np.ndarray) -> tuple[np.ndarray, float]:
    """float32 -> (E4M3 bytes, descale): descale = max|x| / 448 (a float32),
    bytes = x / descale rounded to nearest even by PyTorch's float8_e4m3fn
    conversion, so that bytes * descale approximates x."""
    import torch
    amax = float(np.max(np.abs(x))) if x.size else 1.0
    ds = float(np.float32(amax / 448.0 if amax > 0 else 1.0))
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / np.float32(ds))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), ds


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> the 16-bit storage array (float16, or uint16 bf16 bits)."""
    if dtype == F16:
        return x.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass
class Inputs:
    q: np.ndarray          # [B, Hq, Nq, D]   float16 or uint16 (bf16 bits)
    k: np.ndarray          # [B, Hkv, Nkv, D]
    v: np.ndarray          # [B, Hkv, Nkv, Dv]
    dtype: str
    seed: int
    k_offset: np.ndarray | None = None   # float32 [D], already folded into k
    rows: np.ndarray | None = None       # int64 [Hq, R] sampled query rows
    q_descale: float = 1.0               # FP8: values are bytes * descale
    k_descale: float = 1.0
    v_descale: float = 1.0


def make_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, D: int,
                dtype: str, seed: int = 0, k_offset_std: float | None = None,
                sampled_rows: int | None = None, Dv: int | None = None) -> Inputs:
    """Draw q, k, v iid N(0,1) (float32), in that order, from PCG64(seed);
    v has Dv columns (default D).  For FP8 each tensor is quantised with
    its own descale factor (quantize_fp8).

    With ``k_offset_std`` a per-channel offset c = std*z, z ~ N(0,1) of shape
    [D], is drawn next and added to every key row in float32 before rounding.
    With ``sampled_rows`` = R, each query head then draws R-2 distinct interior
    rows (rows 0 and Nq-1 are always included), sorted.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ds = {}

    def store(name, x):
        if dtype == FP8:
            b, ds[name] = quantize_fp8(x)
            return b
        return to_storage(x, dtype)
    q = rng.standard_normal((B, Hq, Nq, D), dtype=np.float32)
    qs = store("q", q)
    del q
    k = rng.standard_normal((B, Hkv, Nkv, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nkv, D if Dv is None else Dv), dtype=np.float32)
    off = None
    if k_offset_std is not None:
        off = (np.float32(k_offset_std)
               * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
        k += off
    ks = store("k", k)
    del k
    vs = store("v", v)
    del v
    rows = None
    if sampled_rows is not None:
        rows = sample_rows(rng, Hq, Nq, sampled_rows)
    return Inputs(q=qs, k=ks, v=vs, dtype=dtype, seed=seed, k_offset=off,
                  rows=rows, q_descale=ds.get("q", 1.0), k_descale=ds.get("k", 1.0),
                  v_descale=ds.get("v", 1.0))


def make_dout(x: Inputs, seed: int | None = None) -> np.ndarray:
    """The gradient arriving at the output for backward tests: iid N(0,1) of
    the output's shape (q's, with v's head dimension), rounded to the input
    type, from its own PCG64 stream (keyed on [seed, 1], so q, k and v are
    unaffected)."""
    s = x.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64([s, 1]))
    shape = tuple(x.q.shape[:3]) + (x.v.shape[3],)
    return to_storage(rng.standard_normal(shape, dtype=np.float32), x.dtype)


def sample_rows(rng: np.random.Generator, Hq: int, Nq: int, R: int) -> np.ndarray:
    """Per head: rows 0 and Nq-1 plus R-2 distinct interior rows, sorted."""
    if Nq <= R:
        return np.tile(np.arange(Nq, dtype=np.int64), (Hq, 1))
    out = np.empty((Hq, R), dtype=np.int64)
    for h in range(Hq):
        mid = rng.choice(Nq - 2, R - 2, replace=False) + 1
        out[h] = np.sort(np.concatenate([[0, Nq - 1], mid]))
    return out


def make_workload_inputs(w: Workload, seed: int = 0,
                         sampled_rows: int | None = None) -> Inputs:
    R = sampled_rows if sampled_rows is not None else w.sampled_rows
    return make_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.dtype, seed=seed,
                       k_offset_std=w.k_offset_std, sampled_rows=R, Dv=w.Dv)


# ---------------------------------------------------------------------------
# The chunked feed-forward block (FFN chunking, the post's second memory
# saver): token rows x [N, Dm], w1 [F, Dm], b1 [F], w2 [Dm, F], b2 [Dm].
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    name: str
    N: int
    Dm: int
    F: int
    dtype: str
    chunk_rows: int = 0
    note: str = ""

    @property
    def flops(self) -> float:
        """Algorithmic flops of the two products: 4 N Dm F."""
        return 4.0 * self.N * self.Dm * self.F

    def describe(self) -> str:
        return (f"N={self.N} Dm={self.Dm} F={self.F} {self.dtype} "
                f"chunk={self.chunk_rows or 'library'}")


# The 17K-token 480p video of the post's "The problem" through the FFN of a
# 14B-parameter video DiT (model width 5120, hidden width 13824).
FFN_WORKLOADS: dict[str, FfnWorkload] = {
    "dit-ffn-17160": FfnWorkload(name="dit-ffn-17160", N=17160, Dm=5120, F=13824, dtype=BF16,
                                 note="video-DiT feed-forward block, 17K tokens"),
}


@dataclasses.dataclass
class FfnInputs:
    x: np.ndarray     # [N, Dm] 16-bit storage
    w1: np.ndarray    # [F, Dm]
    b1: np.ndarray    # [F]
    w2: np.ndarray    # [Dm, F]
    b2: np.ndarray    # [Dm]
    dtype: str


def make_ffn_inputs(N: int, Dm: int, F: int, dtype: str, seed: int = 0) -> FfnInputs:
    """x iid N(0,1); w1 N(0, 1/Dm), w2 N(0, 1/F) (unit-variance outputs);
    biases N(0, 0.1^2); drawn in that order from PCG64(seed), float32, then
    rounded to the 16-bit type."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((N, Dm), dtype=np.float32)
    w1 = rng.standard_normal((F, Dm), dtype=np.float32) * np.float32(1.0 / math.sqrt(Dm))
    b1 = rng.standard_normal(F, dtype=np.float32) * np.float32(0.1)
    w2 = rng.standard_normal((Dm, F), dtype=np.float32) * np.float32(1.0 / math.sqrt(F))
    b2 = rng.standard_normal(Dm, dtype=np.float32) * np.float32(0.1)
    return FfnInputs(*(to_storage(a, dtype) for a in (x, w1, b1, w2, b2)), dtype=dtype)
