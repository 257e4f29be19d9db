"""Named synthetic workloads.

Shapes follow the model families the pages evaluate (Llama 3.2 1B, Qwen3-8B,
Qwen-R1 32B / Qwen2.5-32B heads; atlas.scime.ai summary, "Key results" and
"Experimental setup"), the 16-token delay window ("Measured effects"), the
32K-context envelope ("Limitations") and the 8x compression ratio (chatpaper.ai
abstract).  The accuracy benchmarks the pages run on these models are not
used: seeded Gaussian activations and logits stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                  # "decode" or "prefill"
    batch: int
    kv_heads: int
    group: int                 # query heads per KV head
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    context: int               # prompt length (decode) or sequence length (prefill)
    steps: int = 0             # decode steps after the prompt
    evict_rate: float | None = 0.5   # fraction marked for eviction; None = per-unit draw
    beta_rate: tuple | None = None   # (a, b): per-unit rate ~ Beta(a, b)
    window: int = 16
    compact_every: int = 16
    prompt_chunk: int = 4096   # prompt appended in chunks of this many tokens
    replicas: int = 1          # independent caches rotated to defeat the 256 MB MALL
    warmup: int = 0
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.group

    @property
    def units(self) -> int:
        return self.batch * self.kv_heads


WORKLOADS = {
    # parity-only tiny case: 1 sequence, 2 KV heads x group 2, fp32, 512-token prompt + 64 steps
    "tiny_f32": Workload(
        name="tiny_f32", kind="decode", batch=1, kv_heads=2, group=2, head_dim=64,
        dtype="f32", context=512, steps=64, evict_rate=0.5, prompt_chunk=512,
        seed=1000,
    ),
    # Llama-3.2-1B-shaped layer at 4x compression
    "llama1b_cr4": Workload(
        name="llama1b_cr4", kind="decode", batch=16, kv_heads=8, group=4, head_dim=64,
        dtype="bf16", context=4096, steps=256, evict_rate=0.75, prompt_chunk=4096,
        replicas=16, seed=2000,
    ),
    # Qwen3-8B-shaped layer at 8x compression: the headline decode workload
    "qwen3_8b_cr8": Workload(
        name="qwen3_8b_cr8", kind="decode", batch=64, kv_heads=8, group=4, head_dim=128,
        dtype="bf16", context=32768, steps=200, evict_rate=0.875, prompt_chunk=4096,
        replicas=4, warmup=20, seed=3000,
    ),
    # the headline shape with float32 keys and values (twice the bytes per retained entry)
    "qwen3_8b_cr8_f32": Workload(
        name="qwen3_8b_cr8_f32", kind="decode", batch=64, kv_heads=8, group=4, head_dim=128,
        dtype="f32", context=32768, steps=32, evict_rate=0.875, prompt_chunk=4096,
        replicas=2, warmup=5, seed=3200,
    ),
    # same shape, nothing evicted (compression ratio 1): the dense control
    "qwen3_8b_cr1": Workload(
        name="qwen3_8b_cr1", kind="decode", batch=64, kv_heads=8, group=4, head_dim=128,
        dtype="bf16", context=32768, steps=20, evict_rate=0.0, prompt_chunk=4096,
        replicas=1, warmup=5, seed=3100,
    ),
    # Qwen2.5-32B heads, 4 prompts x 8 threads, per-unit rate ~ Beta(7, 1): ragged lengths
    "qwen32b_width": Workload(
        name="qwen32b_width", kind="decode", batch=32, kv_heads=8, group=5, head_dim=128,
        dtype="bf16", context=32768, steps=32, evict_rate=None, beta_rate=(7.0, 1.0),
        prompt_chunk=4096, replicas=1, warmup=5, seed=4000,
    ),
    # masked prefill, 8192 tokens, 8x compression
    "prefill_8k": Workload(
        name="prefill_8k", kind="prefill", batch=4, kv_heads=8, group=4, head_dim=128,
        dtype="bf16", context=8192, evict_rate=0.875, seed=5000,
    ),
    # masked prefill of the Llama-3.2-1B-shaped layer (head_dim 64, 4x compression): the
    # prompts of the llama1b_cr4 batch, 4096 tokens each
    "prefill_4k_d64": Workload(
        name="prefill_4k_d64", kind="prefill", batch=16, kv_heads=8, group=4, head_dim=64,
        dtype="bf16", context=4096, evict_rate=0.75, seed=5100,
    ),
}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
