"""Workload shapes: the parameter lists and unit tables of the configurations
the step is measured and checked on.  Shapes only -- no arithmetic.

Units are FSDP wrapping units ("ZeRO and FSDP sharding", Implementation notes:
wrap at transformer-block granularity); a unit's numel is the sum of its
parameters' numels in the order listed.
"""
from __future__ import annotations

from dataclasses import dataclass, field

HIDDEN_GPT2L = 1280
VOCAB_GPT2L = 50304   # the token-id range of the GPT-2 Large runs on "ZeRO: Three Ledgers"
CTX_GPT2L = 1024


def gpt2_block(h: int = HIDDEN_GPT2L):
    """One GPT-2 transformer block with hidden h and a 4h MLP, in order:
    ln_1 (w, b), attention qkv (W, b), attention projection (W, b),
    ln_2 (w, b), MLP fc (W, b), MLP projection (W, b)."""
    return [
        ("ln_1.weight", (h,)), ("ln_1.bias", (h,)),
        ("attn.qkv.weight", (3 * h, h)), ("attn.qkv.bias", (3 * h,)),
        ("attn.proj.weight", (h, h)), ("attn.proj.bias", (h,)),
        ("ln_2.weight", (h,)), ("ln_2.bias", (h,)),
        ("mlp.fc.weight", (4 * h, h)), ("mlp.fc.bias", (4 * h,)),
        ("mlp.proj.weight", (h, 4 * h)), ("mlp.proj.bias", (h,)),
    ]


def gpt2_large_units():
    """36 units totalling 774,090,240 parameters: unit 0 holds the token and
    position embeddings and block 0, units 1-34 one block each, unit 35 the
    last block and the final LayerNorm.  The output head is tied to the token
    embedding, so it adds no parameters."""
    units = []
    for b in range(36):
        ps = [(f"h.{b}.{n}", s) for n, s in gpt2_block()]
        if b == 0:
            ps = [("wte.weight", (VOCAB_GPT2L, HIDDEN_GPT2L)), ("wpe.weight", (CTX_GPT2L, HIDDEN_GPT2L))] + ps
        if b == 35:
            ps = ps + [("ln_f.weight", (HIDDEN_GPT2L,)), ("ln_f.bias", (HIDDEN_GPT2L,))]
        units.append(ps)
    return units


def llama8b_block(h: int = 4096, kv: int = 1024, ffn: int = 14336):
    """One Llama-style block with grouped-query attention (8 KV heads of 128):
    attention norm, q, k, v, o, FFN norm, gate, up, down."""
    return [
        ("attn_norm.weight", (h,)),
        ("q.weight", (h, h)), ("k.weight", (kv, h)), ("v.weight", (kv, h)), ("o.weight", (h, h)),
        ("ffn_norm.weight", (h,)),
        ("gate.weight", (ffn, h)), ("up.weight", (ffn, h)), ("down.weight", (h, ffn)),
    ]


def llama8b_units():
    """34 units totalling 8,030,261,248 parameters: 32 blocks of 218,112,000,
    the token embedding [128256 x 4096], and the untied output head with the
    final norm.  Every unit divides by 64."""
    units = [[(f"layers.{b}.{n}", s) for n, s in llama8b_block()] for b in range(32)]
    units.append([("tok_embeddings.weight", (128256, 4096))])
    units.append([("output.weight", (128256, 4096)), ("norm.weight", (4096,))])
    return units


def numel_of(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def unit_numels(units) -> list[int]:
    return [sum(numel_of(s) for _, s in u) for u in units]


def param_shapes(units) -> list[tuple]:
    """Every parameter's shape, in unit order (one unit per parameter)."""
    return [tuple(s) for u in units for _, s in u]


def row_lengths(shapes) -> list[int]:
    """Row length of each parameter for the dim-0 (row-aligned) layout: the
    product of the trailing dimensions, 1 for a vector."""
    return [numel_of(s[1:]) if len(s) > 1 else 1 for s in shapes]


@dataclass(frozen=True)
class Reshard:
    """A checkpoint reshard: one destination rank's shard of one fp32 state
    array, from a flat layout of FSDP units (from_ranks) to a row-aligned,
    one-unit-per-parameter layout (to_ranks)."""
    name: str
    units: tuple              # unit -> ((name, shape), ...) of the source layout
    from_ranks: int
    to_ranks: int
    dst_rank: int
    dtype: str                # "f32" (master, m, v) or "bf16" (parameters)
    seed: int = 1350
    description: str = ""


def _frozen(units):
    return tuple(tuple((n, tuple(s)) for n, s in u) for u in units)


RESHARDS = {
    "gpt2l_reshard": Reshard(
        "gpt2l_reshard", _frozen(gpt2_large_units()), 8, 4, 1, "f32",
        description="GPT-2-Large-sized fp32 state: 36 flat block units at N=8 -> 436 "
                    "per-parameter dim-0 units at N=4, rank 1's shard (193.6M elements)"),
    "llama8b_reshard": Reshard(
        "llama8b_reshard", _frozen(llama8b_units()), 64, 32, 5, "f32",
        description="8B Llama-shaped fp32 state: 34 flat block units at N=64 -> 291 "
                    "per-parameter dim-0 units at N=32, rank 5's shard (about 251M elements)"),
}


@dataclass(frozen=True)
class Workload:
    name: str
    n_ranks: int
    unit_numel: tuple
    rank: int                 # -1: every rank's shards (the all-gathered view)
    grad_dtype: str           # "bf16" or "f32"
    grad_index: str           # "global" (each rank's full gradient) or "local" (RS chunks)
    out_index: str            # "global" (all-gather slots) or "local" (bf16 shard, ZeRO-3)
    steps: int
    hyper: dict = field(default_factory=dict)
    grad_dist: str = "normal"     # "normal" or "student_t3"
    grad_scale: float = 1e-3
    master_std: float = 0.02
    clip_max_norm: float | None = None
    seed: int = 1337
    description: str = ""


GPT_HYPER = dict(lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
TOY_HYPER = dict(lr=0.01, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)

WORKLOADS = {
    "toy": Workload(
        "toy", 4, (1000,), -1, "f32", "global", "global", 50, TOY_HYPER, seed=1338,
        description="the pages' ZeRO-2 toy: N=4, P=1000, w0=0, rank r's gradient w - t_r with "
                    "t_r[i] = (7i + 13r) mod 11, 50 steps"),
    "gpt2l_block": Workload(
        "gpt2l_block", 8, tuple(unit_numels([gpt2_block()])), -1, "bf16", "global", "global", 10,
        GPT_HYPER, seed=1339,
        description="one FSDP unit shaped like a GPT-2 Large block (19,677,440 params), N=8, "
                    "all 8 shards, bf16 grads ~N(0,1e-3), fp32 master ~N(0,0.02), 10 steps"),
    "gpt2l": Workload(
        "gpt2l", 8, tuple(unit_numels(gpt2_large_units())), -1, "bf16", "global", "global", 10,
        GPT_HYPER, seed=1340,
        description="GPT-2-Large-sized model: 36 units, 774,090,240 params, N=8 simulated ranks' "
                    "bf16 gradient buffers resident, every shard stepped, bf16 out in the "
                    "all-gather slots"),
    "llama8b_z3": Workload(
        "llama8b_z3", 64, tuple(unit_numels(llama8b_units())), 0, "bf16", "local", "local", 10,
        GPT_HYPER, seed=1341,
        description="ZeRO-3 shard of an 8B Llama-shaped model at N=64: rank 0's "
                    "125,472,832-element shard, 64 bf16 reduce-scatter chunks summed per element"),
    "llama8b_z3_clip": Workload(
        "llama8b_z3_clip", 64, tuple(unit_numels(llama8b_units())), 0, "bf16", "local", "local",
        10, GPT_HYPER, grad_dist="student_t3", clip_max_norm=1.0, seed=1342,
        description="as llama8b_z3 plus global-norm clipping at max_norm 1.0 with Student-t(3) "
                    "x 1e-3 gradients"),
}
