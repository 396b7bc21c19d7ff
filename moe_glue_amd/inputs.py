"""Seeded synthetic inputs for the MoE glue path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no routing, no activation, no accumulation).  Both the HIP
path and the CPU oracle consume the arrays it returns, so parity never depends
on the generator itself.

Every tensor is drawn from its own counter-keyed stream,
``SeedSequence([seed, tensor_id, chunk])``, in fixed chunks of ``CHUNK``
elements.  The values therefore do not depend on which other tensors are drawn,
on the number of worker threads, or on the order the chunks finish in.

bf16 tensors are returned as ``uint16`` arrays of raw bf16 bits: an fp32
N(0,1) draw rounded to the nearest bf16, ties to even.

The five workloads are the shapes of the MoE layers named on the pages: a tiny
case, a Qwen3-30B-A3B-shaped prefill batch (the local TP=1 deployment that the
"CuTeDSL at Perplexity" page's MoE section names, and the model of the
FlashInfer CUTLASS-MoE page's results), a decode batch at the same shape, a
DeepSeek-V3-shaped layer with a per-expert router bias, and a skewed routing
case with T=1023 (the odd token count the vLLM test parametrisation uses).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk

# Stream ids: one per tensor, fixed forever (changing them changes every input).
_X, _LOGITS, _BIAS, _RANK, _TIES, _H, _Y, _W, _EXTRA = range(9)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int          # tokens
    H: int          # hidden size
    E: int          # experts
    k: int          # experts per token
    I: int          # expert intermediate size (GEMM1 output is 2*I wide: gate | up)
    bias_std: float = 0.0   # >0: per-expert router bias ~ N(0, bias_std)
    zipf_s: float = 0.0     # >0: per-expert log-Zipf offset folded into the logits
    tie_frac: float = 0.0   # fraction of rows that get an injected exact tie

    @property
    def R(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "Config":
        return dataclasses.replace(self, name=f"{self.name}_T{T}", T=T)


CONFIGS = {
    "tiny": Config("tiny", T=16, H=256, E=8, k=2, I=128),
    "qwen3_30b_a3b": Config("qwen3_30b_a3b", T=4096, H=2048, E=128, k=8, I=768),
    "decode": Config("decode", T=32, H=2048, E=128, k=8, I=768),
    "deepseek_v3": Config("deepseek_v3", T=8192, H=7168, E=256, k=8, I=2048, bias_std=0.5),
    "skewed": Config("skewed", T=1023, H=4096, E=64, k=6, I=1408, zipf_s=1.2, tie_frac=0.01),
}
CONFIG_ORDER = ["tiny", "qwen3_30b_a3b", "decode", "deepseek_v3", "skewed"]


def _normal_f32(seed: int, stream: int, n: int, threads: int = 8) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // CHUNK))

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        if lo < hi:
            rng = np.random.default_rng(np.random.SeedSequence([seed, stream, c]))
            rng.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(threads, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return raw bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, stream: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return f32_to_bf16_bits(_normal_f32(seed, stream, n)).reshape(shape)


def make_x(cfg: Config, seed: int) -> np.ndarray:
    """Token activations x, bf16 bits [T, H], N(0,1)."""
    return normal_bf16(seed, _X, (cfg.T, cfg.H))


def make_logits(cfg: Config, seed: int):
    """Router logits fp32 [T, E] and the optional per-expert bias fp32 [E].

    * base: N(0,1).
    * zipf_s > 0: add -s*ln(rank_e), rank a seeded permutation of 1..E (the
      log of a Zipf(s) pmf over experts), so a few experts are hot.
    * tie_frac > 0: round(tie_frac*T) seeded rows get an exact tie.  Of those
      rows, taken in ascending order, the even-positioned ones copy the k-th
      largest logit onto the (k+1)-th largest (a tie at the selection
      boundary); the odd-positioned ones copy the largest onto the second
      largest (a tie inside the selected set, so only slot order changes).
    * bias_std > 0: bias ~ N(0, bias_std) in fp32.
    """
    T, E, k = cfg.T, cfg.E, cfg.k
    logits = _normal_f32(seed, _LOGITS, T * E).reshape(T, E)
    if cfg.zipf_s > 0.0:
        rng = np.random.default_rng(np.random.SeedSequence([seed, _RANK, 0]))
        rank = rng.permutation(E) + 1
        offset = -cfg.zipf_s * np.log(rank.astype(np.float64))
        logits = (logits.astype(np.float64) + offset[None, :]).astype(np.float32)
    if cfg.tie_frac > 0.0 and T > 0:
        n = int(round(cfg.tie_frac * T))
        rng = np.random.default_rng(np.random.SeedSequence([seed, _TIES, 0]))
        rows = np.sort(rng.choice(T, size=min(n, T), replace=False))
        for i, t in enumerate(rows):
            order = np.argsort(-logits[t].astype(np.float64), kind="stable")
            if i % 2 == 0 and k < E:
                logits[t, order[k]] = logits[t, order[k - 1]]
            elif E >= 2:
                logits[t, order[1]] = logits[t, order[0]]
    bias = None
    if cfg.bias_std > 0.0:
        bias = (np.float32(cfg.bias_std) * _normal_f32(seed, _BIAS, E)).astype(np.float32)
    return np.ascontiguousarray(logits, dtype=np.float32), bias


def tie_rows(cfg: Config, seed: int) -> np.ndarray:
    """Row indices that make_logits injected ties into (empty if none)."""
    if cfg.tie_frac <= 0.0 or cfg.T == 0:
        return np.zeros(0, dtype=np.int64)
    n = int(round(cfg.tie_frac * cfg.T))
    rng = np.random.default_rng(np.random.SeedSequence([seed, _TIES, 0]))
    return np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False))


def make_h(cfg: Config, seed: int) -> np.ndarray:
    """GEMM1 output stand-in, bf16 bits [T*k, 2I]: gate in columns [0,I), up in [I,2I)."""
    return normal_bf16(seed, _H, (cfg.R, 2 * cfg.I))


def make_y(cfg: Config, seed: int) -> np.ndarray:
    """GEMM2 output stand-in, bf16 bits [T*k, H]."""
    return normal_bf16(seed, _Y, (cfg.R, cfg.H))


def make_weights(T: int, k: int, seed: int) -> np.ndarray:
    """Arbitrary positive fp32 routing weights [T, k] (not normalised)."""
    return (np.abs(_normal_f32(seed, _W, T * k)) + np.float32(0.05)).reshape(T, k).astype(np.float32)


def make_inputs(cfg: Config, seed: int, parts=("x", "logits", "h", "y")) -> dict:
    out = {"cfg": cfg, "seed": seed}
    if "x" in parts:
        out["x"] = make_x(cfg, seed)
    if "logits" in parts:
        out["logits"], out["bias"] = make_logits(cfg, seed)
    if "h" in parts:
        out["h"] = make_h(cfg, seed)
    if "y" in parts:
        out["y"] = make_y(cfg, seed)
    return out


# ---------------------------------------------------------------- edge-case logits
def quantized_logits(T: int, E: int, seed: int, step: float = 0.5, span: int = 3) -> np.ndarray:
    """Logits on a coarse grid {-span*step..span*step}: many exact ties per row."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _EXTRA, 1]))
    q = rng.integers(-span, span + 1, size=(T, E))
    return (q.astype(np.float32) * np.float32(step)).astype(np.float32)


def signed_zero_logits(T: int, E: int, seed: int) -> np.ndarray:
    """Rows mixing +0.0, -0.0 and a few negative values: -0 and +0 compare equal."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _EXTRA, 2]))
    choice = rng.integers(0, 3, size=(T, E))
    vals = np.where(choice == 0, np.float32(0.0), np.where(choice == 1, np.float32(-0.0), np.float32(-1.0)))
    return vals.astype(np.float32)


def constant_logits(T: int, E: int, value: float = 0.25) -> np.ndarray:
    return np.full((T, E), np.float32(value), dtype=np.float32)


def wide_logits(T: int, E: int, seed: int, scale: float = 30.0) -> np.ndarray:
    """Large-spread logits: weights far below 1 ulp of the leading weight occur."""
    return (np.float32(scale) * _normal_f32(seed, _EXTRA, T * E)).reshape(T, E).astype(np.float32)


def describe(cfg: Config) -> str:
    extra = []
    if cfg.bias_std:
        extra.append(f"bias~N(0,{cfg.bias_std})")
    if cfg.zipf_s:
        extra.append(f"zipf_s={cfg.zipf_s}")
    if cfg.tie_frac:
        extra.append(f"ties={cfg.tie_frac:g}")
    s = f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I}"
    return s + (" " + " ".join(extra) if extra else "")


__all__ = ["Config", "CONFIGS", "CONFIG_ORDER", "make_inputs", "make_x", "make_logits", "make_h", "make_y",
           "make_weights", "f32_to_bf16_bits", "bf16_bits_to_f32", "quantized_logits", "signed_zero_logits",
           "constant_logits", "wide_logits", "tie_rows", "describe"]
