"""Seeded synthetic inputs for the MoE-layer forward path.

This module is shared by the oracle side and the HIP side of every test and by
the benchmark.  It only draws and shapes input tensors; it contains none of the
layer's arithmetic (no routing, no permutation, no FFN, no combine).

Workloads follow the model shapes that the pages name for expert-parallel MoE
serving (Mixtral 8x7B, DeepSeek-V3, Qwen3-MoE; "Expert Parallelism: MoE model
parallel split", §1 and §4, and "Expert parallelism for MoE serving",
overview), with the sizes of one GPU's share.  No trained weights exist here, so
every tensor is a seeded random draw:

* activations x ~ N(0, 1);
* router, gate and up projections ~ N(0, 1/H); down projections ~ N(0, 1/I);
* draws are fp32 and, for bf16 workloads, rounded to bf16 (round to nearest
  even) before either side sees them;
* an optional router bias is a log-Zipf prior over experts:
  b_e = ln p_{e+1}, p_r = r^-s / sum_{r'=1..E} r'^-s, which skews expert load the
  way the hot-expert discussion of "LLM MoE Expert Parallel production practice"
  (step 1, expert load profile) describes;
* an optional per-token routing budget k_t is drawn uniformly from a set of
  budgets (request-level elastic k, MoE-Prism summary §2B).
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
DT_F32 = 0
DT_BF16 = 1

SEED_ROOT = 0x4D6F45

# tensor tags for seed derivation
TAG_X, TAG_WR, TAG_WG, TAG_WU, TAG_WD, TAG_K, TAG_SG, TAG_SU, TAG_SD, TAG_LOGITS, TAG_MISC = range(11)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    hidden: int
    experts: int
    inter: int
    top_k: int                       # k, or k_max when k_choices is set
    score: int = SCORE_SOFTMAX
    renormalize: int = 1
    routed_scale: float = 1.0
    num_groups: int = 1
    topk_groups: int = 1
    group_topn: int = 0
    capacity_factor: float = 0.0     # <= 0: no capacity limit
    shared_inter: int = 0
    dtype: int = DT_BF16
    zipf_s: float = 0.0              # 0: no router bias
    k_choices: Optional[Sequence[int]] = None

    def with_tokens(self, t: int) -> "LayerConfig":
        return dataclasses.replace(self, tokens=int(t))

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DT_F32 else 2


# The five workloads.  Index order is fixed (it enters the seeds).
CONFIGS: Dict[str, LayerConfig] = {
    # tiny fp32 layer: the size the oracle finishes in seconds
    "tiny_fp32": LayerConfig("tiny_fp32", 256, 512, 8, 1024, 2, dtype=DT_F32),
    # Mixtral-8x7B-shaped prefill and decode layers
    "mixtral_prefill": LayerConfig("mixtral_prefill", 4096, 4096, 8, 14336, 2),
    "mixtral_decode": LayerConfig("mixtral_decode", 64, 4096, 8, 14336, 2),
    # DeepSeek-V3-shaped layer: 256 routed experts + 1 shared, sigmoid scoring,
    # 8 groups / 4 kept, top-8, gates renormalised then scaled by 2.5
    "deepseek_v3": LayerConfig("deepseek_v3", 8192, 7168, 256, 2048, 8, score=SCORE_SIGMOID,
                               routed_scale=2.5, num_groups=8, topk_groups=4, group_topn=2,
                               shared_inter=2048, zipf_s=1.1),
    # Qwen3-MoE-shaped skewed layer: per-token k in {2,4,6,8}, capacity 1.25
    "qwen3_skewed": LayerConfig("qwen3_skewed", 16384, 2048, 128, 768, 8, capacity_factor=1.25,
                                zipf_s=1.2, k_choices=(2, 4, 6, 8)),
}
CONFIG_ORDER = ["tiny_fp32", "mixtral_prefill", "mixtral_decode", "deepseek_v3", "qwen3_skewed"]


def seed_for(cfg_name: str, tag: int, salt: int = 0) -> int:
    """A 63-bit seed from (root, workload name, tensor tag, salt)."""
    h = hashlib.sha256(f"{SEED_ROOT}:{cfg_name}:{tag}:{salt}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, dtype: int, device, seed: int) -> torch.Tensor:
    """fp32 N(0, std^2) draw, rounded to bf16 (RNE) when dtype is bf16."""
    t = torch.randn(*shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if dtype == DT_BF16:
        t = t.to(torch.bfloat16)
    return t


def log_zipf_bias(E: int, s: float) -> np.ndarray:
    """b_e = ln p_{e+1} with p_r proportional to r^-s over ranks 1..E (fp32)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-s)
    return np.log(w / w.sum()).astype(np.float32)


def make_layer_inputs(cfg: LayerConfig, device="cpu", salt: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """All tensors of one layer call, on `device`.

    Layouts (row-major, K contiguous, as nn.Linear stores them):
    x [T,H]; w_router [E,H]; bias [E] fp32; k_per_token [T] int32;
    w_gate, w_up [E,I,H]; w_down [E,H,I]; shared: [Is,H], [Is,H], [H,Is].
    """
    T, H, E, I = cfg.tokens, cfg.hidden, cfg.experts, cfg.inter
    n = cfg.name
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal((T, H), 1.0, cfg.dtype, device, seed_for(n, TAG_X, salt))
    out["w_router"] = normal((E, H), 1.0 / math.sqrt(H), cfg.dtype, device, seed_for(n, TAG_WR, salt))
    out["bias"] = (torch.from_numpy(log_zipf_bias(E, cfg.zipf_s)).to(device) if cfg.zipf_s > 0 else None)
    if cfg.k_choices:
        g = _gen("cpu", seed_for(n, TAG_K, salt))
        choices = torch.tensor(list(cfg.k_choices), dtype=torch.int32)
        idx = torch.randint(0, len(choices), (T,), generator=g)
        out["k_per_token"] = choices[idx].to(device)
    else:
        out["k_per_token"] = None
    out["w_gate"] = normal((E, I, H), 1.0 / math.sqrt(H), cfg.dtype, device, seed_for(n, TAG_WG, salt))
    out["w_up"] = normal((E, I, H), 1.0 / math.sqrt(H), cfg.dtype, device, seed_for(n, TAG_WU, salt))
    out["w_down"] = normal((E, H, I), 1.0 / math.sqrt(I), cfg.dtype, device, seed_for(n, TAG_WD, salt))
    if cfg.shared_inter > 0:
        Is = cfg.shared_inter
        out["ws_gate"] = normal((Is, H), 1.0 / math.sqrt(H), cfg.dtype, device, seed_for(n, TAG_SG, salt))
        out["ws_up"] = normal((Is, H), 1.0 / math.sqrt(H), cfg.dtype, device, seed_for(n, TAG_SU, salt))
        out["ws_down"] = normal((H, Is), 1.0 / math.sqrt(Is), cfg.dtype, device, seed_for(n, TAG_SD, salt))
    else:
        out["ws_gate"] = out["ws_up"] = out["ws_down"] = None
    return out


def make_logits(T: int, E: int, device="cpu", seed: int = 1, bias: Optional[np.ndarray] = None,
                tie_fraction: float = 0.0) -> torch.Tensor:
    """Router logits [T,E] fp32 for routing-only cases.

    N(0,1) draws plus an optional bias row.  With tie_fraction > 0, that share
    of tokens gets exact ties: random experts copy the value of another expert
    of the same token (and some tokens get several equal maxima).
    """
    g = _gen("cpu", seed)
    l = torch.randn(T, E, generator=g, dtype=torch.float32)
    if bias is not None:
        l += torch.from_numpy(bias)[None, :]
    if tie_fraction > 0 and E > 1:
        nt = max(1, int(T * tie_fraction))
        rows = torch.randperm(T, generator=g)[:nt]
        for i, t in enumerate(rows.tolist()):
            ncopy = 1 + (i % 4)
            src = int(torch.randint(0, E, (1,), generator=g))
            if i % 3 == 0:      # tie at the top: copy the row maximum
                src = int(torch.argmax(l[t]))
            dst = torch.randint(0, E, (ncopy,), generator=g)
            l[t, dst] = l[t, src].clone()
        # a few rows that are entirely equal
        for t in rows[: max(1, nt // 16)].tolist():
            l[t, :] = l[t, 0].clone()
    return l.to(device)


def make_k_per_token(T: int, choices: Sequence[int], seed: int, device="cpu") -> torch.Tensor:
    g = _gen("cpu", seed)
    c = torch.tensor(list(choices), dtype=torch.int32)
    return c[torch.randint(0, len(c), (T,), generator=g)].to(device)


def to_numpy_raw(t: Optional[torch.Tensor]):
    """Host numpy view of a tensor: bf16 as its raw uint16 bits, else as is."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    return (a.astype(np.uint32) << 16).view(np.float32)
