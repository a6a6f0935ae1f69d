"""Seeded synthetic workloads for the Block AttnRes depth-aggregation path.

This module is shared by the HIP path's drivers/benchmark and by the test
harness that feeds the CPU oracle.  It holds *only* workload shapes and random
number generation: no RMSNorm, no scores, no softmax, no sums of sources.
Every other module may import it; it imports neither the oracle nor the HIP
binding.

Workloads (sizes as given for the method's deployment shapes; the pages
describe the K3 layout as 93 decoder layers = 186 sublayers in 8 blocks,
seven of 24 sublayers and a tail of 18 -- "Kimi K3 模型结构 (4)", block
partition Q&A):

* ``tiny_block_f32``     T=64,     d=256,  L=8 in 2 blocks of 4, fp32
* ``full_bf16``          T=4096,   d=1024, L=16, every sublayer its own source
* ``decode_block_bf16``  T=256,    d=7168, one block of 24 sublayers on top of
                         the embedding and 7 completed block sums
* ``prefill_chunk_bf16`` T=16384,  d=7168, 186 sublayers in 7x24 + 18
* ``long_prefill_bf16``  T=131072, same depth layout, streamed in 16K chunks

Randomness: every tensor is drawn from ``torch`` generators seeded from
``(workload seed, tensor kind, index, 1024-token block)``.  Drawing per
1024-token block makes a token's values independent of how the sequence is
chunked, so a chunked run sees bit-identical inputs to an unchunked one.
Sublayer outputs and the embedding are drawn on the device that will hold
them; the small parameter tensors are drawn on the host and copied, so they
are identical on every device.  Values are rounded to the storage dtype
(round-to-nearest-even for bf16) before anybody sees them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import torch

TOKEN_BLOCK = 1024  # tokens per seeding block (divides every chunk length used)

# tensor-kind tags for seed derivation
_K_EMB, _K_V, _K_GIVEN, _K_W, _K_G, _K_GAMMA, _K_SCALE = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens
    d: int                      # hidden width
    block_sizes: tuple          # sublayers per block computed in this pass
    dtype: str                  # storage dtype: "f32" or "bf16"
    seed: int
    full: bool = False          # every sublayer is its own source (N = L)
    n_given: int = 0            # completed block sums supplied as inputs
    final_site: bool = True     # aggregate b_0..b_N once more at the end
    unit_gains: bool = False    # key gain g and PreNorm gain gamma fixed at 1
    v_scale: str = "loguniform_0.5_8"   # per-sublayer scale law
    given_scale: str = "loguniform_1_16"
    eps: float = 1e-6
    chunk: Optional[int] = None  # tokens per chunk for streamed prefill

    @property
    def L(self) -> int:
        return int(sum(self.block_sizes))

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS: Dict[str, Workload] = {
    "tiny_block_f32": Workload("tiny_block_f32", T=64, d=256, block_sizes=(4, 4),
                               dtype="f32", seed=1001, unit_gains=True),
    "full_bf16": Workload("full_bf16", T=4096, d=1024, block_sizes=(1,) * 16,
                          dtype="bf16", seed=1002, full=True, v_scale="linear_1_4"),
    "decode_block_bf16": Workload("decode_block_bf16", T=256, d=7168, block_sizes=(24,),
                                  dtype="bf16", seed=1003, n_given=7, final_site=False,
                                  unit_gains=True),
    "prefill_chunk_bf16": Workload("prefill_chunk_bf16", T=16384, d=7168,
                                   block_sizes=(24,) * 7 + (18,), dtype="bf16", seed=1004),
    "long_prefill_bf16": Workload("long_prefill_bf16", T=131072, d=7168,
                                  block_sizes=(24,) * 7 + (18,), dtype="bf16", seed=1004,
                                  chunk=16384),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller test shapes)."""
    return dataclasses.replace(w, **changes)


def _seed(*parts: int) -> int:
    # 64-bit FNV-1a over the integer parts: a fixed, documented derivation
    h = 0xCBF29CE484222325
    for p in parts:
        for b in int(p).to_bytes(8, "little", signed=False):
            h ^= b
            h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_rows(seed: int, kind: int, index: int, t0: int, t1: int, d: int,
                device, out_dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) rows for tokens [t0, t1), drawn per 1024-token block so that a
    token's values do not depend on the chunking.  Returns ``out_dtype``."""
    dev = torch.device(device)
    out = torch.empty((t1 - t0, d), dtype=out_dtype, device=dev)
    b0, b1 = t0 // TOKEN_BLOCK, (t1 - 1) // TOKEN_BLOCK
    for b in range(b0, b1 + 1):
        lo, hi = b * TOKEN_BLOCK, (b + 1) * TOKEN_BLOCK
        g = _gen(dev, _seed(seed, kind, index, b))
        blk = torch.randn((TOKEN_BLOCK, d), generator=g, device=dev, dtype=torch.float32)
        s, e = max(lo, t0), min(hi, t1)
        out[s - t0:e - t0] = blk[s - lo:e - lo].to(out_dtype)
        del blk
    return out


def _scales(w: Workload, kind: int, count: int, law: str) -> List[float]:
    if law.startswith("linear_"):
        a, b = (float(x) for x in law.split("_")[1:])
        if count == 1:
            return [a]
        return [a + (b - a) * i / (count - 1) for i in range(count)]
    if law.startswith("loguniform_"):
        a, b = (float(x) for x in law.split("_")[1:])
        g = _gen("cpu", _seed(w.seed, kind, 0, 0))
        u = torch.rand(count, generator=g, dtype=torch.float64)
        return [math.exp(math.log(a) + (math.log(b) - math.log(a)) * float(x)) for x in u]
    raise ValueError(law)


def sublayer_scales(w: Workload) -> List[float]:
    return _scales(w, _K_SCALE, w.L, w.v_scale)


def given_scales(w: Workload) -> List[float]:
    return _scales(w, _K_GIVEN + 100, w.n_given, w.given_scale)


def params(w: Workload, device="cpu") -> Dict[str, torch.Tensor]:
    """Per-site parameters, fp32, drawn on the host: ``w``, ``g`` (key gain)
    of shape [L+1, d] (row L is the final site's) and ``gamma`` (PreNorm gain)
    of shape [L, d].  Pseudo-queries ~ N(0, 0.02^2); gains ~ U(0.8, 1.2) or 1."""
    L, d = w.L, w.d
    q = torch.randn((L + 1, d), generator=_gen("cpu", _seed(w.seed, _K_W, 0, 0)),
                    dtype=torch.float32) * 0.02
    if w.unit_gains:
        g = torch.ones((L + 1, d), dtype=torch.float32)
        gam = torch.ones((L, d), dtype=torch.float32)
    else:
        g = 0.8 + 0.4 * torch.rand((L + 1, d), generator=_gen("cpu", _seed(w.seed, _K_G, 0, 0)),
                                   dtype=torch.float32)
        gam = 0.8 + 0.4 * torch.rand((L, d), generator=_gen("cpu", _seed(w.seed, _K_GAMMA, 0, 0)),
                                     dtype=torch.float32)
    return {"w": q.to(device), "g": g.to(device), "gamma": gam.to(device)}


def embedding(w: Workload, t0: int, t1: int, device) -> torch.Tensor:
    """b_0 rows for tokens [t0, t1): N(0,1) in the storage dtype."""
    return normal_rows(w.seed, _K_EMB, 0, t0, t1, w.d, device, w.torch_dtype)


def sublayer_output(w: Workload, l: int, t0: int, t1: int, device,
                    scales: Optional[Sequence[float]] = None) -> torch.Tensor:
    """Synthetic output v_l of sublayer l (1-based) for tokens [t0, t1):
    s_l * N(0,1), rounded to the storage dtype."""
    s = (scales if scales is not None else sublayer_scales(w))[l - 1]
    x = normal_rows(w.seed, _K_V, l, t0, t1, w.d, device, torch.float32)
    return (x * s).to(w.torch_dtype)


def given_block(w: Workload, n: int, t0: int, t1: int, device,
                scales: Optional[Sequence[float]] = None) -> torch.Tensor:
    """Completed block sum b_n (1-based) supplied as an input (decode-shaped
    step): s_n * N(0,1) in the storage dtype."""
    s = (scales if scales is not None else given_scales(w))[n - 1]
    x = normal_rows(w.seed, _K_GIVEN, n, t0, t1, w.d, device, torch.float32)
    return (x * s).to(w.torch_dtype)


def sample_tokens(T: int, count: int) -> List[int]:
    """Deterministic token sample: evenly spaced, always including 0 and T-1."""
    if count >= T:
        return list(range(T))
    idx = sorted({round(i * (T - 1) / (count - 1)) for i in range(count)})
    return idx
