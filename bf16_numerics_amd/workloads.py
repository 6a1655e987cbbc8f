"""Synthetic workloads: tensor tables and seeded input generators.

This module holds inputs only -- tensor lists in flat-buffer order, the
per-tensor decay flag the training loop would pass, hyperparameters and seeded
random draws.  It contains none of the optimizer's arithmetic, so both the HIP
path and the CPU oracle can be fed from it.

Shapes follow the model dimensions named for each workload.  The decay flag is
set for 2-D tensors (embeddings and weight matrices) and cleared for 1-D ones
(LayerNorm / RMSNorm weights and biases), the split the llm.c chapter
("04 · 多 GPU 与混合精度", §2.2) describes.
"""
from dataclasses import dataclass, field
import math

import numpy as np

SEED = 1337


@dataclass(frozen=True)
class HParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    bias_correction: bool = True
    max_norm: float = 1.0


@dataclass
class Workload:
    name: str
    tensors: list                      # [(name, shape)] in flat-buffer order
    hparams: HParams = field(default_factory=HParams)
    world: int = 1                     # ZeRO-1 shard count
    rank: int = 0                      # shard timed / checked by default
    steps: int = 10
    grad_kind: str = "normal"          # normal | per_tensor_loguniform | constant
    grad_std: float = 1e-3
    grad_const: float = 0.0
    param_kind: str = "normal"         # normal | uniform
    param_std: float = 0.02
    param_range: tuple = (0.5, 2.0)

    @property
    def n(self) -> int:
        return sum(math.prod(s) for _, s in self.tensors)

    def entries(self):
        """(offset, numel, flags) triples; flags bit 0 = weight decay (2-D tensor)."""
        out, off = [], 0
        for _, shape in self.tensors:
            numel = math.prod(shape)
            out.append((off, numel, 1 if len(shape) == 2 else 0))
            off += numel
        return out

    def shard(self, rank=None):
        r = self.rank if rank is None else rank
        per = self.n // self.world
        return r * per, (r + 1) * per


def gpt2_tensors(V, T, C, L):
    t = [("wte", (V, C)), ("wpe", (T, C))]
    for l in range(L):
        t += [
            (f"h{l}.ln1w", (C,)), (f"h{l}.ln1b", (C,)),
            (f"h{l}.qkvw", (C, 3 * C)), (f"h{l}.qkvb", (3 * C,)),
            (f"h{l}.attprojw", (C, C)), (f"h{l}.attprojb", (C,)),
            (f"h{l}.ln2w", (C,)), (f"h{l}.ln2b", (C,)),
            (f"h{l}.fcw", (C, 4 * C)), (f"h{l}.fcb", (4 * C,)),
            (f"h{l}.fcprojw", (4 * C, C)), (f"h{l}.fcprojb", (C,)),
        ]
    t += [("lnfw", (C,)), ("lnfb", (C,))]
    return t


def llama_tensors(V, d, ffn, L):
    t = [("embed", (V, d))]
    for l in range(L):
        t += [
            (f"l{l}.attn_norm", (d,)),
            (f"l{l}.wq", (d, d)), (f"l{l}.wk", (d, d)), (f"l{l}.wv", (d, d)), (f"l{l}.wo", (d, d)),
            (f"l{l}.ffn_norm", (d,)),
            (f"l{l}.w1", (ffn, d)), (f"l{l}.w2", (d, ffn)), (f"l{l}.w3", (ffn, d)),
        ]
    t += [("norm", (d,)), ("lm_head", (V, d))]
    return t


def tiny() -> Workload:
    """2-layer GPT, d=32: 28 tensors, 29,568 parameters; grads ~N(0, 1e-3); 16 steps."""
    return Workload("tiny_gpt_d32", gpt2_tensors(64, 64, 32, 2), steps=16, grad_std=1e-3)


def gpt2_124m() -> Workload:
    """GPT-2 124M (V 50304, T 1024, C 768, L 12): 148 tensors, 124,475,904 parameters."""
    return Workload("gpt2_124m", gpt2_tensors(50304, 1024, 768, 12), steps=10,
                    grad_kind="per_tensor_loguniform")


def gpt2_1p5b_shard() -> Workload:
    """One 1/8 ZeRO-1 shard of GPT-2 1.5B (L 48, C 1600, V 50304, T 1024):
    n = 1,557,686,400, shard = 194,710,800.  Rank 1 is the default: both of
    its ends fall inside tensors."""
    return Workload("gpt2_1p5b_shard", gpt2_tensors(50304, 1024, 1600, 48), world=8, rank=1,
                    steps=50, grad_kind="per_tensor_loguniform")


def stall16m() -> Workload:
    """Small-update stall: one 2^24 tensor, no decay, P ~ U(0.5, 2), G = -2^-10,
    lr = 0.1 * 2^-7 (a tenth of a bf16 step at 1), 1000 steps."""
    return Workload("stall16m", [("w", (1 << 24,))],
                    hparams=HParams(lr=0.1 * 2.0 ** -7, weight_decay=0.0),
                    steps=1000, grad_kind="constant", grad_const=-(2.0 ** -10),
                    param_kind="uniform")


def llama7b() -> Workload:
    """Llama-style 7B (L 32, d 4096, ffn 11008, V 32000, untied head): 291 tensors,
    6,738,415,616 parameters; grads ~N(0, 1e-4); 20 steps."""
    return Workload("llama7b", llama_tensors(32000, 4096, 11008, 32), steps=20, grad_std=1e-4)


WORKLOADS = {"tiny_gpt_d32": tiny, "gpt2_124m": gpt2_124m, "gpt2_1p5b_shard": gpt2_1p5b_shard,
             "stall16m": stall16m, "llama7b": llama7b}


# --------------------------------------------------------------------------
# Seeded generators (torch on any device; values are bf16 bit patterns as
# int16/uint16 storage, or float32).
# --------------------------------------------------------------------------

def _gen(torch, device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def tensor_ranges(w: Workload, begin: int, end: int):
    """(local_lo, local_hi, tensor_index) for each tensor piece inside [begin, end)."""
    out = []
    for k, (off, numel, _) in enumerate(w.entries()):
        lo, hi = max(off, begin), min(off + numel, end)
        if lo < hi:
            out.append((lo - begin, hi - begin, k))
    return out


def grad_stds(w: Workload, seed=SEED):
    """Per-tensor grad std: constant, or log-uniform in [1e-5, 1e-2] drawn once."""
    if w.grad_kind == "per_tensor_loguniform":
        rs = np.random.default_rng(seed ^ 0x5EED)
        u = rs.uniform(math.log(1e-5), math.log(1e-2), size=len(w.tensors))
        return [float(math.exp(x)) for x in u]
    return [w.grad_std] * len(w.tensors)


def init_state(torch, w: Workload, begin: int, end: int, device, seed=SEED, master=True):
    """Initial (P bf16, M f32 or None, m f32, v f32) over global [begin, end)."""
    count = end - begin
    g = _gen(torch, device, seed * 1000003 + begin % 1000003)
    if w.param_kind == "uniform":
        lo, hi = w.param_range
        p32 = torch.empty(count, dtype=torch.float32, device=device).uniform_(lo, hi, generator=g)
    else:
        p32 = torch.empty(count, dtype=torch.float32, device=device).normal_(0.0, w.param_std, generator=g)
    P = p32.to(torch.bfloat16)
    del p32
    M = P.to(torch.float32) if master else None
    m = torch.zeros(count, dtype=torch.float32, device=device)
    v = torch.zeros(count, dtype=torch.float32, device=device)
    return P, M, m, v


def init_params_into(torch, w: Workload, begin: int, P, M=None, seed=SEED, chunk=1 << 27):
    """Initial bf16 params for global [begin, begin + len(P)) written into the
    existing tensor P (and their fp32 copy into M), chunk by chunk, so that no
    full-size temporary is needed.  Same distribution as init_state; each
    chunk has its own seeded generator."""
    count = P.numel()
    for c0 in range(0, count, chunk):
        c1 = min(count, c0 + chunk)
        g = _gen(torch, P.device, (seed * 1000003 + begin + c0) % (1 << 62))
        tmp = torch.empty(c1 - c0, dtype=torch.float32, device=P.device)
        if w.param_kind == "uniform":
            tmp.uniform_(w.param_range[0], w.param_range[1], generator=g)
        else:
            tmp.normal_(0.0, w.param_std, generator=g)
        P[c0:c1] = tmp.to(torch.bfloat16)
        if M is not None:
            M[c0:c1] = P[c0:c1].to(torch.float32)
    return P


def fill_grads(torch, w: Workload, G, begin: int, step: int, seed=SEED, stds=None):
    """Write step `step`'s bf16 grads for global [begin, begin + len(G)) into G."""
    end = begin + G.numel()
    if w.grad_kind == "constant":
        G.fill_(w.grad_const)
        return G
    g = _gen(torch, G.device, (seed * 7919 + step * 104729 + begin) % (1 << 62))
    stds = grad_stds(w, seed) if stds is None else stds
    tmp = torch.empty(G.numel(), dtype=torch.float32, device=G.device)
    tmp.normal_(0.0, 1.0, generator=g)
    if w.grad_kind == "normal":
        tmp.mul_(stds[0])
    else:
        for lo, hi, k in tensor_ranges(w, begin, end):
            tmp[lo:hi].mul_(stds[k])
    G.copy_(tmp.to(torch.bfloat16))
    del tmp
    return G


def bf16_bits_numpy(torch, t):
    """Host copy of a bf16 tensor as uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(torch, bits, device="cpu"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
