"""Synthetic workloads: parameter-shape lists, layouts and value recipes.

Input recipe only -- nothing here performs any step of the update.  Used by
the tests, the smoke check and the benchmark to build inputs with the shapes
and value distributions of the five shard workloads:

  flat1m     one flat tensor of 1,048,576 parameters, one bucket, N_d = 4
  gpt2s      GPT-2-small parameter list (148 tensors), 25 MiB buckets, N_d = 8
  accum1p3b  one flat tensor of 1.3e9 parameters, one bucket, N_d = 8, with
             4 no_sync micro-batches per rank before the step
  llama8b    Llama-3-8B parameter list (291 tensors), 25 MiB buckets, N_d = 8
  llama70b   Llama-2/3-70B parameter list (723 tensors), 25 MiB buckets,
             N_d = 64, ZeRO-3 in-place output
  llama70b_t the same list cut into 12,500,000-element buckets, which leaves a
             zero-padded tail in every bucket slice of the last rank
  gpt2s_fsdp2    GPT-2-small list in the per-parameter dim-0 layout, N_d = 8
                 (the 50257-row embedding leaves padding rows on the last rank)
  llama8b_fsdp2  Llama-3-8B list in the per-parameter dim-0 layout, N_d = 8,
                 ZeRO-3 in place

Distributions are named (kind, scale): "normal" N(0, scale) with scale the
standard deviation, "absnormal" |N(0, scale)|, "student_t3" Student-t with 3
degrees of freedom times scale, "normal_zeros" N(0, scale) with 1 % of the
draws replaced by exact +0, "zero" all zeros.
"""
from __future__ import annotations

from dataclasses import dataclass, field

MiB25 = 25 * 1024 * 1024 // 2        # 25 MiB of bf16 = 13,107,200 elements


def gpt2_small_shapes():
    """GPT-2 small in forward order: wte, wpe, 12 blocks, final LayerNorm."""
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    shapes = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(12):
        p = f"h{i}."
        shapes += [
            (p + "ln_1.weight", (d,)), (p + "ln_1.bias", (d,)),
            (p + "attn.c_attn.weight", (d, 3 * d)), (p + "attn.c_attn.bias", (3 * d,)),
            (p + "attn.c_proj.weight", (d, d)), (p + "attn.c_proj.bias", (d,)),
            (p + "ln_2.weight", (d,)), (p + "ln_2.bias", (d,)),
            (p + "mlp.c_fc.weight", (d, ff)), (p + "mlp.c_fc.bias", (ff,)),
            (p + "mlp.c_proj.weight", (ff, d)), (p + "mlp.c_proj.bias", (d,)),
        ]
    shapes += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return shapes


def llama_shapes(n_layers, d, kv, ff, vocab):
    """Llama-style decoder in forward order: embedding, blocks, norm, head."""
    shapes = [("embed_tokens", (vocab, d))]
    for i in range(n_layers):
        p = f"layers.{i}."
        shapes += [
            (p + "input_layernorm", (d,)),
            (p + "q_proj", (d, d)), (p + "k_proj", (kv, d)), (p + "v_proj", (kv, d)),
            (p + "o_proj", (d, d)),
            (p + "post_attention_layernorm", (d,)),
            (p + "gate_proj", (ff, d)), (p + "up_proj", (ff, d)), (p + "down_proj", (d, ff)),
        ]
    shapes += [("norm", (d,)), ("lm_head", (vocab, d))]
    return shapes


def numel_of(shapes):
    out = []
    for _, s in shapes:
        n = 1
        for k in s:
            n *= k
        out.append(n)
    return out


@dataclass
class Workload:
    name: str
    numel: list
    cap: int            # bucket capacity in elements; <= 0 means one bucket
    n_d: int
    rank: int
    grad_layout: str    # "flat": each rank hands a padded flat buffer; "compact": its slice
    out_mode: str       # "ag_slot" (ZeRO-1/2) or "shard" (ZeRO-3, in place)
    t_first: int        # 1-based step index of the first step
    n_steps: int
    grad: tuple
    master: tuple
    exp_avg: tuple
    exp_avg_sq: tuple
    n_micro: int = 0    # > 0: grads come from no_sync accumulation of n_micro micro-batches
    micro_grad: tuple = ("zero", 0.0)
    hp: dict = field(default_factory=lambda: dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                                                  weight_decay=0.1))
    shapes: list = None
    rows: list = None   # per-tensor dim-0 sizes: the per-parameter (FSDP2) layout

    @property
    def psi(self):
        return sum(self.numel)


def _llama8b():
    return llama_shapes(32, 4096, 1024, 14336, 128256)


def _llama70b():
    return llama_shapes(80, 8192, 1024, 28672, 128256)


def get(name: str) -> Workload:
    if name == "flat1m":
        return Workload("flat1m", [1 << 20], 0, 4, 3, "flat", "ag_slot", 1, 10,
                        ("normal", 1e-3), ("normal", 0.02), ("zero", 0.0), ("zero", 0.0))
    if name == "gpt2s":
        sh = gpt2_small_shapes()
        return Workload("gpt2s", numel_of(sh), MiB25, 8, 7, "flat", "ag_slot", 1, 10,
                        ("normal", 1e-3), ("normal", 0.02), ("zero", 0.0), ("zero", 0.0),
                        shapes=sh)
    if name == "accum1p3b":
        return Workload("accum1p3b", [1_300_000_000], 0, 8, 7, "compact", "ag_slot", 101, 1,
                        ("zero", 0.0), ("normal", 0.02), ("normal", 1e-4), ("absnormal", 1e-6),
                        n_micro=4, micro_grad=("normal", 2e-3))
    if name == "llama8b":
        sh = _llama8b()
        return Workload("llama8b", numel_of(sh), MiB25, 8, 7, "compact", "ag_slot", 1, 10,
                        ("student_t3", 1e-3), ("normal", 0.02), ("zero", 0.0), ("zero", 0.0),
                        shapes=sh)
    if name in ("llama70b", "llama70b_t"):
        sh = _llama70b()
        cap = MiB25 if name == "llama70b" else 12_500_000
        return Workload(name, numel_of(sh), cap, 64, 63, "compact", "shard", 1001, 1,
                        ("normal_zeros", 1e-3), ("normal", 0.02), ("normal", 1e-4),
                        ("absnormal", 1e-6), shapes=sh)
    if name == "gpt2s_fsdp2":
        sh = gpt2_small_shapes()
        return Workload(name, numel_of(sh), 0, 8, 7, "flat", "ag_slot", 1, 3,
                        ("normal", 1e-3), ("normal", 0.02), ("zero", 0.0), ("zero", 0.0),
                        shapes=sh, rows=[s[1][0] for s in sh])
    if name == "llama8b_fsdp2":
        sh = _llama8b()
        return Workload(name, numel_of(sh), 0, 8, 7, "compact", "shard", 1, 2,
                        ("student_t3", 1e-3), ("normal", 0.02), ("zero", 0.0), ("zero", 0.0),
                        shapes=sh, rows=[s[1][0] for s in sh])
    raise KeyError(name)


NAMES = ("flat1m", "gpt2s", "accum1p3b", "llama8b", "llama70b", "llama70b_t")
DIM0_NAMES = ("gpt2s_fsdp2", "llama8b_fsdp2")
