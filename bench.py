"""DMS decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload qwen3_8b_cr8]
                    [--batch B] [--context T] [--evict-rate R] [--window W]
                    [--compact-every N] [--seed S] [--replicas N]

(The page size is fixed at 64 slots by the library.)  A run with overrides
reports them under config.overrides and no counter-based traffic figure.

A step is one pass of the whole decode hot path for one attention layer over
a batch: decide + append the new token of every (sequence, KV head) unit,
split-K decode attention over the retained entries, and compaction, one
every `compact_every` steps (rotating over the cache replicas, so that each
replica is compacted once every `compact_every` of its own steps).  Steps
rotate over independent cache replicas so that the working set exceeds the
256 MB last-level cache.  All inputs are generated on the GPU before the
timed region, which holds only the steps between two HIP events; per-call
times come from a separate pass over further steps.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import contextlib
import dataclasses
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (matrix and vector), published
METRIC = "DMS decode-attn tokens/s and KV GB/s (% HBM peak) at CR=8, Qwen3-8B shape"
# the other decode workloads, each measured by a short step loop of its own:
# Llama-3.2-1B-shaped heads at CR 4, the Qwen3-8B shape with nothing evicted,
# ragged Qwen2.5-32B-shaped units
DECODE_CONFIGS = ("llama1b_cr4", "qwen3_8b_cr1", "qwen32b_width", "qwen3_8b_cr8_f32")
DEFAULT_WORKLOAD = "qwen3_8b_cr8"
PMC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_qwen3_8b_cr8_traffic.json")
DECODE_SRC = os.path.join(ROOT, "decode_attention_learned_amd", "csrc", "decode_mfma.hip")
PREFILL_SRC = os.path.join(ROOT, "decode_attention_learned_amd", "csrc", "prefill.hip")
PREFILL_F32_SRC = os.path.join(ROOT, "decode_attention_learned_amd", "csrc", "prefill_f32.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def marked(name: str):
    """A roctx range named `name` around a part of the run (torch.cuda.nvtx emits
    roctx ranges on ROCm builds): `rocprofv3 --marker-trace` then places every
    kernel in its leg."""
    import torch

    torch.cuda.nvtx.range_push(name)
    try:
        yield
    finally:
        torch.cuda.nvtx.range_pop()


# workload fields the command line may override, with their flags
OVERRIDES = (("batch", "--batch", int, "sequences in the batch"),
             ("context", "--context", int, "prompt tokens per sequence"),
             ("evict_rate", "--evict-rate", float, "fraction of tokens marked for eviction"),
             ("window", "--window", int, "delay window w (tokens)"),
             ("compact_every", "--compact-every", int, "steps between compactions of a replica"),
             ("seed", "--seed", int, "seed of the synthetic inputs"))


def apply_overrides(w, args):
    """The workload with the command line's overrides applied, and the overrides."""
    over = {f: getattr(args, f) for f, *_ in OVERRIDES if getattr(args, f) is not None}
    if not over:
        return w, {}
    if over.get("batch", 1) < 1 or over.get("context", 1) < 1 or over.get("window", 1) < 1 \
            or over.get("compact_every", 1) < 1:
        raise SystemExit(f"bench.py: overrides must be positive: {over}")
    if not 0.0 <= over.get("evict_rate", 0.0) < 1.0:
        raise SystemExit("bench.py: --evict-rate must lie in [0, 1)")
    if "evict_rate" in over:
        over["beta_rate"] = None          # a fixed rate replaces a per-unit draw
    return dataclasses.replace(w, **over), over


def src_hash(path: str) -> str:
    """Hash of a kernel source's code: comments and whitespace are dropped, so
    that counters taken on it stay valid across documentation edits."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def retained_total(cache) -> tuple[int, int]:
    """(sum over units of |R(t)|, sum of slots in use) from the cache metadata."""
    import torch

    n = cache.n_slots.long()
    maxn = int(n.max().item())
    if maxn == 0:
        return 0, 0
    npg = (maxn + 63) // 64
    pages = cache.page_table[:, :npg].long().clamp(min=0)
    pos = cache.slot_pos[pages].reshape(cache.units, -1)[:, :maxn]
    alpha = cache.slot_alpha[pages].reshape(cache.units, -1)[:, :maxn]
    idx = torch.arange(maxn, device=n.device)[None, :]
    in_use = idx < n[:, None]
    t = (cache.seq_len.long() - 1).repeat_interleave(cache.kv_heads)[:, None]
    live = in_use & ((alpha == 0) | ((t - pos.long()) < cache.window))
    return int(live.sum().item()), int(in_use.sum().item())


def pool_size(w, rates, extra_tokens):
    """(max_pages_per_unit, num_pages) with room for the expected retained set of
    every unit (plus 6 sigma), one prompt chunk in flight and `extra_tokens`."""
    import numpy as np

    keep = 1.0 - rates.reshape(-1)
    mean = w.context * keep + w.window
    sd = np.sqrt(w.context * keep * (1.0 - keep))
    per_unit = np.ceil((mean + 6 * sd + extra_tokens) / 64).astype(np.int64) + w.prompt_chunk // 64 + 2
    per_unit = np.minimum(per_unit, (w.context + extra_tokens) // 64 + 2)
    return int(per_unit.max()), int(per_unit.sum())


def build_replica(w, r, dev, extra_tokens):
    import torch

    import workloads as wl
    from decode_attention_learned_amd import DmsCache

    rates = wl.unit_eviction_rates(w, r)
    max_pages, num_pages = pool_size(w, rates, extra_tokens)
    cache = DmsCache(w.batch, w.kv_heads, w.group, w.head_dim,
                     torch.float32 if w.dtype == "f32" else torch.bfloat16,
                     num_pages=num_pages, max_pages_per_unit=max_pages,
                     window=w.window, device=dev)
    for ci, start in enumerate(range(0, w.context, w.prompt_chunk)):
        n = min(w.prompt_chunk, w.context - start)
        k, v, logit = wl.prompt_chunk_inputs(w, ci, n, device=dev, replica=r, rates=rates)
        cache.append(k, v, logit)
        cache.compact()
        del k, v, logit
    torch.cuda.synchronize()
    if cache.status_word() != 0:
        raise RuntimeError(f"replica {r}: device status {cache.status_word()} while building")
    return cache, rates


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds: float = 12.0, threads: int = 1) -> dict:
    """Time the float64 oracle on host cores on a bounded sample of the same workload:
    one sequence (all its KV heads) with the full context, then decode steps
    (append, attend, compaction every `compact_every` steps) until `seconds` pass.
    BLAS may use `threads` threads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle import dms_oracle as orc

    sample = wl.Workload(**{**{k: v for k, v in w.__dict__.items() if k != "extra"}, "batch": 1})
    rates = wl.unit_eviction_rates(sample)
    units = [orc.UnitCache(sample.window, sample.head_dim, dtype=np.float32)
             for _ in range(sample.kv_heads)]
    scale = 1.0 / math.sqrt(sample.head_dim)
    with threadpool_limits(limits=threads):
        for ci, start in enumerate(range(0, sample.context, sample.prompt_chunk)):
            n = min(sample.prompt_chunk, sample.context - start)
            k, v, logit = wl.prompt_chunk_inputs(sample, ci, n, rates=rates)
            alpha = orc.eviction_decisions(logit.numpy())
            kf, vf = k.float().numpy(), v.float().numpy()
            for h, uc in enumerate(units):
                uc.append(alpha[0, :, h], kf[0, :, h], vf[0, :, h])
                uc.compact()
        steps = 0
        kv_bytes = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            q, k, v, logit = wl.decode_step_inputs(sample, steps, rates=rates)
            alpha = orc.eviction_decisions(logit.numpy())
            qf = q.double().numpy()
            kf, vf = k.float().numpy(), v.float().numpy()
            for h, uc in enumerate(units):
                uc.append(alpha[0, :, h], kf[0, :, h], vf[0, :, h])
                uc.attend(qf[0, h * sample.group:(h + 1) * sample.group], scale)
                kv_bytes += int(uc.live().sum()) * sample.head_dim * 2 * 2  # K and V, bf16
                if (steps + 1) % sample.compact_every == 0:
                    uc.compact()
            steps += 1
        dt = time.perf_counter() - t0
    return {"value": steps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "seconds_per_step": round(dt / steps, 6),
            "kv_gbps": round(kv_bytes / dt / 1e9, 4),
            "sample": f"1 of {w.batch} sequences ({sample.kv_heads} KV heads x G={sample.group}, "
                      f"context {sample.context}), {steps} decode steps in {dt:.1f} s, "
                      f"float64 NumPy with BLAS limited to {threads} thread(s); tokens/s is the "
                      f"same for the full batch (each of its steps is {w.batch} such sequences)"}


def fill_launch_ms(caches, inputs, outs, scale: float, n_launch: int) -> float:
    """Mean duration of the decode launch (dms_decode_attn_fill) with no event
    between launches.  Every replica first takes one more step (reserve, then
    the fill) with its last prepared inputs; then `n_launch` further fill
    launches, rotating over the replicas, run back to back between two events
    on the library's stream (one untimed launch first, so that the stream is
    busy when the start event is recorded).  A repeated fill serves the
    replica's reserved token again with the same inputs: it streams the same
    slots and rewrites the token's slot with the same bytes, so every cache
    ends as after its one step.  An event recorded between launches costs a
    few microseconds of queue time, which per-call events would add to every
    launch."""
    import torch

    replicas = len(caches)
    for r in range(replicas):
        q, k, v, logit = inputs[r][-1]
        caches[r][0].reserve()
        caches[r][0].fill_and_decode(k, v, logit, q, outs[r], scale)

    def launch(n):
        r = n % replicas
        q, k, v, logit = inputs[r][-1]
        caches[r][0].fill_and_decode(k, v, logit, q, outs[r], scale)

    launch(0)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for n in range(1, n_launch + 1):
        launch(n)
    end.record()
    torch.cuda.synchronize()
    if any(c.status_word() for c, _ in caches):
        raise RuntimeError("device status set in the launch pass")
    return start.elapsed_time(end) / n_launch


def _time_calls(fn, iters: int) -> float:
    """Mean milliseconds of fn() over `iters` calls, HIP events on the current stream.

    One untimed call is queued right before the timed ones, so that the stream
    is busy when the first start event is recorded: otherwise the first
    interval would also hold the time the idle GPU waits for the host to
    queue that call's kernels."""
    import torch

    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    fn()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / iters


def gathered_tiles(keep, s_len: int, window: int, block: int = 32, tile: int = 32) -> int:
    """Key tiles the gathered kernel processes, summed over units and query
    blocks: the gathered kept keys up to the block's last query - w, plus the
    dense tiles of the band (q0 - w, last query]."""
    import torch

    csum = torch.cumsum(keep, dim=1)                               # [B, S, Hkv] kept at <= position
    total = 0
    for q0 in range(0, s_len, block):
        i_max = min(s_len, q0 + block) - 1
        x = i_max - window
        n_any = csum[:, x, :] if x >= 0 else torch.zeros_like(csum[:, 0, :])
        ngt = (n_any + tile - 1) // tile
        nb = i_max // tile - max(0, q0 - window + 1) // tile + 1
        total += int(ngt.sum().item()) + nb * keep.shape[0] * keep.shape[2]
    return total


def prefill_cpu_baseline(name: str = "prefill_8k", threads: int = 1) -> dict:
    """Time the float64 oracle's masked prefill (prefill_rows) on the host on a
    bounded sample of the prefill workload: one sequence of the same shape and
    distributions, query rows [0, 512) and [S - 512, S), every query head.  The
    oracle computes each row over all S keys (masked), so its cost per row is
    the same everywhere; the rate is query positions (all heads) per second."""

    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle import dms_oracle as orc

    w = wl.get(name)
    ws = dataclasses.replace(w, batch=1)
    q, k, v, logit = wl.prefill_inputs(ws)
    alpha = orc.eviction_decisions(logit.numpy())
    s_len = w.context
    rows = np.r_[0:512, s_len - 512:s_len]
    qf, kf, vf = q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy()
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        orc.prefill_rows(qf, kf, vf, alpha[0], rows, w.window, 1.0 / math.sqrt(w.head_dim))
        dt = time.perf_counter() - t0
    return {"value": round(len(rows) / dt, 2), "unit": "query positions/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "seconds": round(dt, 3),
            "seconds_per_call_extrapolated": round(dt * s_len / len(rows) * w.batch, 1),
            "sample": f"1 sequence of the {name} shape ({w.q_heads}/{w.kv_heads} heads, D={w.head_dim}, "
                      f"S={s_len}), query rows [0, 512) and [{s_len - 512}, {s_len}) with all heads, "
                      f"float64 NumPy, BLAS limited to {threads} thread(s)"}


def prefill_leg(name: str = "prefill_8k", iters: int = 10, relaxed: bool = True) -> dict:
    """Masked prefill on one prefill workload (default: 8192 tokens, head_dim 128).

    Dense (dms_prefill_attn): causal FLOPs per second of one call (pack pass +
    attention kernel) against the dense bf16 MFMA peak.  Gathered
    (dms_prefill_attn_gathered): the same result; its roofline uses the MFMA
    work it executes (key tiles x 32 queries x heads), and the causal FLOPs
    over its time are reported as the equivalent dense rate."""
    import torch

    import workloads as wl
    from decode_attention_learned_amd import lib, prefill
    from decode_attention_learned_amd.cache import PAGE, _DTYPES

    w = wl.get(name)
    dev = torch.device("cuda:0")
    q, k, v, logit = wl.prefill_inputs(w, device=dev)
    s_len, d = w.context, w.head_dim
    out = torch.empty((w.batch, s_len, w.q_heads, d), dtype=torch.float32, device=dev)
    shape = lib.DmsShape(w.batch, w.kv_heads, w.group, d, PAGE, w.window, 1, 1, _DTYPES[torch.bfloat16])
    ws = torch.empty((lib.prefill_gathered_workspace_bytes(shape, s_len),), dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda: prefill(q, k, v, logit, window=w.window, out=out, workspace=ws), iters)
    ms_g = _time_calls(lambda: prefill(q, k, v, logit, window=w.window, out=out, workspace=ws,
                                       method="gathered"), iters)
    if relaxed:
        noise = wl.logistic_noise(w, device=dev)
        ms_r = _time_calls(lambda: prefill(q, k, v, logit, window=w.window, out=out, workspace=ws,
                                           method="relaxed", noise=noise, temperature=1.0), iters)
    causal = 4.0 * d * s_len * (s_len + 1) / 2 * w.batch * w.q_heads
    # visible (query, key) pairs: |R(i)| = #{j <= i - w : unmarked} + min(w, i + 1), per (b, h)
    keep = (logit <= 0).to(torch.int64)                          # [B, S, Hkv]
    csum = torch.cumsum(keep, dim=1)
    i = torch.arange(s_len, device=dev)
    idx = (i - w.window).clamp(min=-1)
    kept_before = torch.where(idx[None, :, None] >= 0,
                              csum.gather(1, idx.clamp(min=0)[None, :, None].expand_as(csum)),
                              torch.zeros_like(csum))
    pairs = (kept_before + torch.clamp(i + 1, max=w.window)[None, :, None]).sum().item() * w.group
    visible = 4.0 * d * pairs
    tflops = causal / (ms * 1e-3) / 1e12
    # executed MFMA work of the gathered kernel: per key tile and workgroup
    # (32 query positions), QK and PV products over 32 keys x 32 queries x G heads x D
    executed = 4.0 * 32 * 32 * d * w.group * gathered_tiles(keep, s_len, w.window)
    g_tflops = executed / (ms_g * 1e-3) / 1e12
    rec = {
        "workload": name, "batch": w.batch, "seq_len": s_len, "q_heads": w.q_heads,
        "kv_heads": w.kv_heads, "head_dim": d, "evict_rate": w.evict_rate, "window": w.window,
        "ms": round(ms, 4), "causal_tflop": round(causal / 1e12, 4),
        "visible_pair_tflop": round(visible / 1e12, 4),
        "query_positions_per_s": round(w.batch * s_len / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "k_prefill_pack + k_prefill", "achieved": round(tflops, 1),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": prefill_traffic_from_profile("dense", name),
                     "algorithmic_bytes_per_call": prefill_algorithmic_bytes(
                         w.batch, s_len, w.q_heads, w.kv_heads, d),
                     "workspace_bytes_per_call": prefill_workspace_traffic(
                         w.batch, s_len, w.kv_heads, d)},
        "gathered": {
            "ms": round(ms_g, 4), "speedup_vs_dense": round(ms / ms_g, 2),
            "causal_equivalent_tflops": round(causal / (ms_g * 1e-3) / 1e12, 1),
            "executed_tflop": round(executed / 1e12, 4),
            "roofline": {"bound": "mfma",
                         "kernel": "k_sparse_scan + k_sparse_pack + k_prefill_gathered",
                         "achieved": round(g_tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(g_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": prefill_traffic_from_profile("gathered", name)},
        },
    }
    if relaxed:
        rec["relaxed"] = {"ms": round(ms_r, 4), "temperature": 1.0, "noise": "logistic",
                          "causal_tflops": round(causal / (ms_r * 1e-3) / 1e12, 1),
                          "frac": round(causal / (ms_r * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    return rec


def prefill_f32_leg(name: str = "prefill_8k", iters: int = 3) -> dict:
    """Masked prefill of the same workload shape with float32 inputs
    (k_prefill_f32 on v_mfma_f32_16x16x4_f32): causal FLOPs per second against
    the fp32 peak, for the hard rule and the relaxed mask."""
    import torch

    import workloads as wl
    from decode_attention_learned_amd import prefill

    w = dataclasses.replace(wl.get(name), dtype="f32")
    dev = torch.device("cuda:0")
    q, k, v, logit = wl.prefill_inputs(w, device=dev)
    s_len, d = w.context, w.head_dim
    out = torch.empty((w.batch, s_len, w.q_heads, d), dtype=torch.float32, device=dev)
    ws = torch.empty((256,), dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda: prefill(q, k, v, logit, window=w.window, out=out, workspace=ws), iters)
    noise = wl.logistic_noise(w, device=dev)
    ms_r = _time_calls(lambda: prefill(q, k, v, logit, window=w.window, out=out, workspace=ws,
                                       method="relaxed", noise=noise, temperature=1.0), iters)
    causal = 4.0 * d * s_len * (s_len + 1) / 2 * w.batch * w.q_heads
    tf, tf_r = causal / (ms * 1e-3) / 1e12, causal / (ms_r * 1e-3) / 1e12
    return {"workload": name, "dtype": "f32", "batch": w.batch, "seq_len": s_len, "head_dim": d,
            "ms": round(ms, 3), "relaxed_ms": round(ms_r, 3),
            "roofline": {"bound": "mfma", "kernel": f"k_prefill_f32<{d}>", "achieved": round(tf, 1),
                         "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / FP32_PEAK_TFLOPS, 4),
                         "relaxed_frac": round(tf_r / FP32_PEAK_TFLOPS, 4),
                         "traffic": prefill_traffic_from_profile("dense", name, f32=True),
                         "relaxed_traffic": prefill_traffic_from_profile("relaxed", name, f32=True),
                         "algorithmic_bytes_per_call": prefill_algorithmic_bytes(
                             w.batch, s_len, w.q_heads, w.kv_heads, d, in_bytes=4)}}


def chunk_leg(caches, w, dev, n_query: int = 4, rounds: int = 32) -> dict:
    """Chunk queries on the decode workload's caches: every round appends
    n_query tokens to one replica and attends all of them at once
    (dms_decode_attn_multi), compacting each replica every 16 tokens.  The
    K/V of every retained entry is read once per launch of 16 / G queries.
    The rounds are queued back to back (one synchronisation at the end), as a
    serving loop would issue them."""
    import torch

    import workloads as wl

    gen = torch.Generator(device=dev)
    gen.manual_seed(977)
    per_launch = max(1, 16 // w.group)
    launches = (n_query + per_launch - 1) // per_launch
    inputs = []
    for i in range(rounds):
        r = i % len(caches)
        k, v, logit = wl.prompt_chunk_inputs(w, 100000 + i, n_query, device=dev, replica=r,
                                             rates=caches[r][1])
        q = torch.randn((w.batch, n_query, w.q_heads, w.head_dim), generator=gen, device=dev,
                        dtype=torch.float32).to(torch.bfloat16)
        inputs.append((q, k, v, logit))
    torch.cuda.synchronize()
    before = [retained_total(c)[0] for c, _ in caches]
    evs, flags = [], []
    for i in range(rounds):
        cache = caches[i % len(caches)][0]
        q, k, v, logit = inputs[i]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        cache.append(k, v, logit)
        ev[1].record()
        cache.decode_chunk(q)
        ev[2].record()
        compacted = ((i // len(caches) + 1) * n_query) % 16 == 0
        if compacted:
            cache.compact()
        ev[3].record()
        evs.append(ev)
        flags.append(compacted)
    torch.cuda.synchronize()
    after = [retained_total(c)[0] for c, _ in caches]
    if any(c.status_word() for c, _ in caches):
        raise RuntimeError("device status set during the chunk leg")
    warm = len(caches)  # first round per replica is warm-up
    t_app = [e[0].elapsed_time(e[1]) for e in evs[warm:]]
    t_att = [e[1].elapsed_time(e[2]) for e in evs[warm:]]
    t_cmp = [e[2].elapsed_time(e[3]) for e, f in zip(evs[warm:], flags[warm:]) if f]
    att = sum(t_att) / len(t_att)
    app = sum(t_app) / len(t_app)
    cmp_per_round = (sum(t_cmp) / max(1, len(t_cmp))) * n_query / 16
    step = app + att + cmp_per_round
    retained = (sum(before) + sum(after)) / (2 * len(caches))
    bytes_alg = retained * w.head_dim * 2 * 2 * launches
    return {
        "n_query": n_query, "launches_per_call": launches,
        "attn_us": round(att * 1e3, 2), "append_us": round(app * 1e3, 2),
        "tokens_per_s": round(w.batch * n_query / (step * 1e-3), 1),
        "kv_gbps": round(bytes_alg / (att * 1e-3) / 1e9, 1),
        "hbm_frac": round(bytes_alg / (att * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
    }


def shared_prefix_leg(w, dev, threads: int = 8, steps: int = 24) -> dict:
    """Width scaling from shared prompts: the decode workload's B sequences as
    B / threads prompts with `threads` threads each.  One cache holds every
    prompt once per thread (each thread appended it); the other holds it once
    per prompt and shares it (dms_share_prefix).  Same tokens, same outputs;
    reported: pages held and decode-attention time of both."""

    import torch

    import workloads as wl
    from decode_attention_learned_amd import DmsCache

    n_prompts = w.batch // threads
    wp = dataclasses.replace(w, batch=n_prompts)
    rates = wl.unit_eviction_rates(wp)
    max_pages, _ = pool_size(w, wl.unit_eviction_rates(w), steps + 64)
    num_pages = w.units * max_pages
    caches = {m: DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, torch.bfloat16, num_pages=num_pages,
                          max_pages_per_unit=max_pages, window=w.window, device=dev)
              for m in ("copied", "shared")}
    lead = torch.arange(0, w.batch, threads, device=dev)
    for ci, start in enumerate(range(0, w.context, w.prompt_chunk)):
        n = min(w.prompt_chunk, w.context - start)
        k, v, logit = wl.prompt_chunk_inputs(wp, ci, n, device=dev, rates=rates)
        caches["copied"].append(k.repeat_interleave(threads, 0), v.repeat_interleave(threads, 0),
                                logit.repeat_interleave(threads, 0))
        caches["copied"].compact()
        # followers of the shared cache receive marked zero tokens, dropped below
        kz = torch.zeros((w.batch, *k.shape[1:]), dtype=k.dtype, device=dev)
        vz = torch.zeros_like(kz)
        lz = torch.ones((w.batch, *logit.shape[1:]), dtype=logit.dtype, device=dev)
        kz[lead], vz[lead], lz[lead] = k, v, logit
        caches["shared"].append(kz, vz, lz)
        caches["shared"].compact()
        del k, v, logit, kz, vz, lz
    sh = caches["shared"]
    for p_ in range(n_prompts):
        sh.release(p_ * threads + 1, threads - 1)
        sh.share_prefix(p_ * threads, p_ * threads + 1, threads - 1)
    torch.cuda.synchronize()
    held = {m: c.num_pages - int(c.free_top.item()) for m, c in caches.items()}
    if any(c.status_word() for c in caches.values()):
        raise RuntimeError("device status set while building the shared-prefix caches")
    ws = dataclasses.replace(w, context=steps)
    q, k, v, logit = wl.prefill_inputs(ws, device=dev)
    times = {m: [] for m in caches}
    outs = {}
    for t in range(steps):
        for m, c in caches.items():
            c.append(k[:, t:t + 1].contiguous(), v[:, t:t + 1].contiguous(), logit[:, t:t + 1].contiguous())
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            outs[m] = c.decode(q[:, t].contiguous())
            b.record()
            torch.cuda.synchronize()
            if t >= 4:
                times[m].append(a.elapsed_time(b))
            if t % w.compact_every == w.compact_every - 1:
                c.compact()
    same = bool(torch.equal(outs["copied"], outs["shared"]))
    retained, _ = retained_total(caches["copied"])
    bytes_alg = retained * w.head_dim * 2 * 2
    us = {m: 1e3 * sum(x) / len(x) for m, x in times.items()}
    return {
        "prompts": n_prompts, "threads_per_prompt": threads, "context": w.context,
        "pages_copied": held["copied"], "pages_shared": held["shared"],
        "memory_ratio": round(held["copied"] / held["shared"], 2),
        "decode_us_copied": round(us["copied"], 2), "decode_us_shared": round(us["shared"], 2),
        "kv_gbps_algorithmic_shared": round(bytes_alg / (us["shared"] * 1e-6) / 1e9, 1),
        "outputs_identical": same,
    }


def chunked_prefill_leg(name: str = "prefill_8k", chunk: int = 512, iters: int = 5,
                        batch: int | None = None) -> dict:
    """Chunked prefill into a cache: the prefill workload's first S - chunk
    tokens are appended and compacted, then the last `chunk` tokens are
    appended and attend at once (dms_decode_attn_multi, tiled kernel).  The
    same rows as the prefill's last `chunk` query rows.  Reported: time of the
    chunk attention and its rate on the visible (query, key) pairs."""
    import torch

    import workloads as wl
    from decode_attention_learned_amd import DmsCache

    w = wl.get(name)
    if batch is not None:
        w = dataclasses.replace(w, batch=batch)
    dev = torch.device("cuda:0")
    q, k, v, logit = wl.prefill_inputs(w, device=dev)
    s_len, d = w.context, w.head_dim
    head = s_len - chunk
    cache = DmsCache(w.batch, w.kv_heads, w.group, d, torch.bfloat16,
                     max_pages_per_unit=(s_len + 63) // 64 + 2, window=w.window, device=dev)
    cache.append(k[:, :head].contiguous(), v[:, :head].contiguous(), logit[:, :head].contiguous())
    cache.compact()
    cache.append(k[:, head:].contiguous(), v[:, head:].contiguous(), logit[:, head:].contiguous())
    qc = q[:, head:].contiguous()
    out = torch.empty((w.batch, chunk, w.q_heads, d), dtype=torch.float32, device=dev)
    ms = _time_calls(lambda: cache.decode_chunk(qc, out=out), iters)
    # the same call with the minimal workspace: no split of the tiles
    from decode_attention_learned_amd import lib
    small = torch.empty((max(lib.decode_multi_workspace_bytes(cache.shape), 1),), dtype=torch.uint8,
                        device=dev)

    def one_pass():
        lib.check("dms_decode_attn_multi", lib.dms_decode_attn_multi(
            cache.shape, cache.cache, qc, chunk, out, 1.0 / math.sqrt(d), small, small.numel(),
            torch.cuda.current_stream().cuda_stream))

    ms_one = _time_calls(one_pass, iters)
    if cache.status_word():
        raise RuntimeError("device status set in the chunked-prefill leg")
    keep = (logit <= 0).to(torch.int64)
    csum = torch.cumsum(keep, dim=1)
    i = torch.arange(head, s_len, device=dev)
    kept_before = csum[:, i - w.window, :]
    pairs = (kept_before + w.window).sum().item() * w.group
    flops = 4.0 * d * pairs
    return {"batch": w.batch, "chunk": chunk, "context_before": head, "ms": round(ms, 4),
            "ms_without_split": round(ms_one, 4),
            "split_workspace_bytes": lib.decode_multi_split_workspace_bytes(cache.shape, chunk),
            "visible_pair_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "tokens_per_s": round(w.batch * chunk / (ms * 1e-3), 1)}


def decode_config_leg(name: str, steps: int = 64, warmup: int = 8, n_ev: int = 32) -> dict:
    """The decode step on another decode workload (its own shape, key/value dtype,
    eviction rates and replica count), measured like the headline: `steps` steps
    between two events (reserve + decode with the token, compaction every
    `compact_every` steps per replica, round-robin over the replicas), then
    `n_ev` back-to-back decode launches (fill_launch_ms) for its time and KV
    rate (on float32 caches the call also holds the launch that writes the
    token)."""
    import torch

    import workloads as wl

    w = wl.get(name)
    dev = torch.device("cuda:0")
    replicas, every = w.replicas, w.compact_every
    # one more input per replica for the launch pass
    per_rep = (warmup + steps + replicas - 1) // replicas + 1
    caches = [build_replica(w, r, dev, per_rep + every + 64) for r in range(replicas)]
    inputs = [[wl.decode_step_inputs(w, j, device=dev, replica=r, rates=caches[r][1])
               for j in range(per_rep)] for r in range(replicas)]
    outs = [torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
            for _ in range(replicas)]
    scale = 1.0 / math.sqrt(w.head_dim)

    def step(i):
        r, j = i % replicas, i // replicas
        cache = caches[r][0]
        q, k, v, logit = inputs[r][j]
        cache.reserve()
        cache.fill_and_decode(k, v, logit, q, outs[r], scale)
        if (i + 1) % every == 0:
            caches[((i + 1) // every - 1) % replicas][0].compact()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    before = [retained_total(c) for c, _ in caches]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(warmup, warmup + steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    if any(c.status_word() for c, _ in caches):
        raise RuntimeError(f"{name}: device status set")
    dec_ms = fill_launch_ms(caches, inputs, outs, scale, n_ev)
    after = [retained_total(c) for c, _ in caches]
    retained = sum(a[0] + b[0] for a, b in zip(before, after)) / (2 * replicas)
    bytes_alg = retained * w.head_dim * 2 * (4 if w.dtype == "f32" else 2)
    kv_gbps = bytes_alg / (dec_ms * 1e-3) / 1e9
    del caches, inputs, outs
    torch.cuda.empty_cache()
    return {"workload": name, "batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads,
            "head_dim": w.head_dim, "kv_dtype": w.dtype, "context": w.context, "evict_rate": w.evict_rate,
            "replicas": replicas, "steps": steps, "ms_per_step": round(ms_step, 4),
            "tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
            "decode_attn_us": round(dec_ms * 1e3, 2),
            "retained_per_unit": round(retained / w.units, 1),
            "kv_gbps": round(kv_gbps, 1), "hbm_frac": round(kv_gbps / HBM_PEAK_GBPS, 4)}


def _profile_record(path: str, src: str):
    """A committed rocprofv3 counter summary, or None if there is none or the
    kernel source changed since it was taken."""
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != src_hash(src):
        return None
    return rec


def traffic_from_profile(bytes_alg_per_launch: float):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary."""
    rec = _profile_record(PMC_FILE, DECODE_SRC)
    return rec.get("hbm_bytes_per_launch") if rec else None


def prefill_traffic_from_profile(method: str = "dense", workload: str = "prefill_8k", f32: bool = False):
    """HBM bytes per prefill call of `method` ("dense", "gathered" or "relaxed":
    every kernel of the call) on `workload` from the committed rocprofv3 counter
    summary (bf16 inputs, or float32 with `f32`), or None if there is none."""
    name = f"prefill_f32_{workload.removeprefix('prefill_')}" if f32 else workload
    rec = _profile_record(os.path.join(ROOT, "profiles", f"{name}_traffic.json"),
                          PREFILL_F32_SRC if f32 else PREFILL_SRC)
    return rec.get(method, {}).get("hbm_bytes_per_call") if rec else None


def prefill_algorithmic_bytes(batch: int, seq_len: int, q_heads: int, kv_heads: int, d: int,
                              in_bytes: int = 2) -> int:
    """Bytes a masked prefill call must move through HBM whatever its design
    (inputs of `in_bytes` per element, fp32 output): Q, K, V and the logits in
    once, O out once."""
    kv = batch * seq_len * kv_heads * d * in_bytes * 2   # K and V
    logits = batch * seq_len * kv_heads * 4
    q = batch * seq_len * q_heads * d * in_bytes
    o = batch * seq_len * q_heads * d * 4
    return kv + logits + q + o


def prefill_workspace_traffic(batch: int, seq_len: int, kv_heads: int, d: int) -> int:
    """Bytes the dense call's own design adds on top (overhead, not algorithmic):
    the pack pass writes the packed tiles, their zeroed far copy and the masks,
    and the attention kernel reads them back."""
    kv = batch * seq_len * kv_heads * d * 2 * 2
    masks = batch * seq_len * kv_heads * 4
    return 2 * (2 * kv + masks)


def calibrate(gib: float) -> dict:
    """Plain device-to-device copies and a full read (sum) of a buffer of known size.

    The copy is the reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE
    counters (a copy of N bytes reads N and writes N), and both give the
    bandwidth this machine reaches with library kernels."""
    import torch

    n = int(gib * (1 << 30)) // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_()
    b = torch.empty_like(a)
    # the read: a sum over the same bytes viewed as fp32 (every value finite:
    # its high half is a finite bf16), which torch reduces with wide loads
    a32 = a.view(torch.float32)
    for _ in range(2):
        b.copy_(a)
        a32.sum()
    torch.cuda.synchronize()
    reps = 5
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    for _ in range(reps):
        a32.sum()
    e2.record()
    torch.cuda.synchronize()
    nbytes = 2 * n
    copy_s = e0.elapsed_time(e1) / reps * 1e-3
    sum_s = e1.elapsed_time(e2) / reps * 1e-3
    return {"calibration": "device copy and full read", "bytes": nbytes,
            "copy_read_plus_write_gbps": round(2 * nbytes / copy_s / 1e9, 1),
            "sum_read_gbps": round(nbytes / sum_s / 1e9, 1),
            "copy_launches": reps + 2, "sum_launches": reps + 2}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--replicas", type=int, default=None)
    for field, flag, kind, what in OVERRIDES:
        ap.add_argument(flag, dest=field, type=kind, default=None, help=f"override the workload's {what}")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate", type=float, default=None, metavar="GIB",
                    help="only run the copy/read calibration on a buffer of GIB GiB")
    ap.add_argument("--no-prefill", action="store_true", help="skip the masked-prefill leg")
    ap.add_argument("--prefill-only", action="store_true", help="only run the masked-prefill leg")
    ap.add_argument("--prefill-d64-only", action="store_true",
                    help="only run the head_dim 64 masked-prefill leg (4096 tokens)")
    ap.add_argument("--prefill-f32-only", action="store_true",
                    help="only run the float32 masked-prefill leg")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunk-query leg")
    ap.add_argument("--append-launch", action="store_true",
                    help="time the step as dms_append + dms_decode_attn (the token written by its "
                         "own launch) instead of dms_append_reserve + dms_decode_attn_fill")
    ap.add_argument("--no-share", action="store_true", help="skip the shared-prefix leg")
    ap.add_argument("--chunked-prefill-only", action="store_true",
                    help="only run the chunked-prefill leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode step on the other decode workloads")
    ap.add_argument("--configs-only", action="store_true",
                    help="only run the decode step on the other decode workloads")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the DMS path here runs on a single MI355X "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate is not None:
        print(json.dumps(calibrate(args.calibrate)), flush=True)
        return
    if args.prefill_only:
        print(json.dumps(prefill_leg()), flush=True)
        return
    if args.prefill_d64_only:
        print(json.dumps(prefill_leg("prefill_4k_d64", relaxed=False)), flush=True)
        return
    if args.prefill_f32_only:
        print(json.dumps(prefill_f32_leg()), flush=True)
        return
    if args.chunked_prefill_only:
        print(json.dumps({"chunked_prefill": chunked_prefill_leg(),
                          "chunked_prefill_one_sequence": chunked_prefill_leg(batch=1)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({n: decode_config_leg(n) for n in DECODE_CONFIGS}), flush=True)
        return
    dev = torch.device("cuda:0")
    w, over = apply_overrides(wl.get(args.workload), args)
    replicas = args.replicas or w.replicas
    every = w.compact_every
    # the breakdown pass: per-call events on every step, at least one compaction
    # of every replica, after the timed window
    n_break = max(64, every * replicas)
    total = args.warmup + args.steps + n_break
    # one more input per replica for the launch pass (fill_launch_ms)
    per_rep = (total + replicas - 1) // replicas + 1
    n_launch = 64
    extra = per_rep + every + 64

    log(f"[bench] building {replicas} replica(s) of {w.name}: B={w.batch} Hkv={w.kv_heads} "
        f"G={w.group} D={w.head_dim} context={w.context}")
    t_build = time.perf_counter()
    with marked("build"):
        caches = [build_replica(w, r, dev, extra) for r in range(replicas)]
    log(f"[bench] built in {time.perf_counter() - t_build:.1f} s")

    inputs = [[wl.decode_step_inputs(w, j, device=dev, replica=r, rates=caches[r][1])
               for j in range(per_rep)] for r in range(replicas)]
    outs = [torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
            for _ in range(replicas)]
    torch.cuda.synchronize()

    scale = 1.0 / math.sqrt(w.head_dim)

    # Global step i runs on replica i % replicas.  Step i: reserve the token's slot
    # (dms_append_reserve), then the decode launch takes the token into the
    # attention and writes it to its page (dms_decode_attn_fill); the same as
    # dms_append + dms_decode_attn.  Every `every`-th global step also compacts
    # one replica, in turn, so each replica is compacted once every `every` of
    # its own steps and any window of steps holds its share of compactions.
    # With `ev`, per-call events are recorded (the breakdown pass only), and
    # `peak` collects pages and slots in use of the replica about to be compacted.
    def step(i, ev=None, peak=None):
        r = i % replicas
        j = i // replicas
        cache = caches[r][0]
        q, k, v, logit = inputs[r][j]
        if ev is not None:
            ev[0].record()
        if args.append_launch:
            cache.append(k, v, logit)
        else:
            cache.reserve()
        if ev is not None:
            ev[1].record()
        if args.append_launch:
            cache.decode(q, out=outs[r], sm_scale=scale)
        else:
            cache.fill_and_decode(k, v, logit, q, outs[r], scale)
        if ev is not None:
            ev[2].record()
        compacted = (i + 1) % every == 0
        if compacted:
            rc = caches[((i + 1) // every - 1) % replicas][0]
            if peak is not None:
                peak.append((rc.num_pages - rc.free_top[0], rc.n_slots.sum()))
            if ev is not None:
                ev[3].record()
            rc.compact()
        if ev is not None:
            ev[4].record()
        return compacted

    with marked("warmup"):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
    before = [retained_total(c) for c, _ in caches]

    # the timed window: the steps alone between two events on the library's stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    n_compact = 0
    with marked("timed steps"):
        start.record()
        for i in range(args.warmup, args.warmup + args.steps):
            n_compact += step(i)
        end.record()
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    after = [retained_total(c) for c, _ in caches]
    status = [c.status_word() for c, _ in caches]
    if any(status):
        raise RuntimeError(f"device status words {status}")

    # breakdown pass: per-call events on further steps of the same caches
    i0 = args.warmup + args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_break)]
    peaks = []
    with marked("breakdown"):
        flags = [step(i0 + i, evs[i], peaks) for i in range(n_break)]
        torch.cuda.synchronize()
    if any(c.status_word() for c, _ in caches):
        raise RuntimeError("device status set in the breakdown pass")
    t_reserve = [e[0].elapsed_time(e[1]) for e in evs]
    t_decode = [e[1].elapsed_time(e[2]) for e in evs]
    t_compact = [e[3].elapsed_time(e[4]) for e, f in zip(evs, flags) if f]
    peak_pages = max(int(p) for p, _ in peaks)
    peak_slots = max(int(n) for _, n in peaks)
    # the decode launch's duration for the roofline: back-to-back launches
    with marked("launch pass"):
        launch_ms = (fill_launch_ms(caches, inputs, outs, scale, n_launch)
                     if not args.append_launch else None)

    ms_step = total_ms / args.steps
    dec_ev_ms = sum(t_decode) / len(t_decode)   # with an event before and after every call
    dec_ms = launch_ms if launch_ms is not None else dec_ev_ms
    res_ms = sum(t_reserve) / len(t_reserve)
    cmp_ms = sum(t_compact) / len(t_compact)
    retained = sum(a[0] + b[0] for a, b in zip(before, after)) / (2 * replicas)
    in_use = sum(a[1] + b[1] for a, b in zip(before, after)) / (2 * replicas)
    elem = 2  # bf16
    bytes_alg = retained * w.head_dim * 2 * elem            # K and V of every retained entry
    bytes_read = in_use * w.head_dim * 2 * elem             # including dead, not yet compacted slots
    kv_gbps = bytes_alg / (dec_ms * 1e-3) / 1e9
    tokens_s = w.batch / (ms_step * 1e-3)
    cr = (w.context + (args.warmup + args.steps / 2) / replicas) * w.units / retained
    dense_tokens = w.units * (w.context + per_rep)

    result = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads,
            "head_dim": w.head_dim, "context": w.context, "evict_rate": w.evict_rate,
            "window": w.window, "compact_every": every, "page_size": 64,
            "replicas": replicas, "kv_dtype": "bf16", "accumulate": "fp32",
            "overrides": over or None,
        },
        "step_calls": ("dms_append + dms_decode_attn" if args.append_launch
                       else "dms_append_reserve + dms_decode_attn_fill") + " + dms_compact every "
                      f"{every} steps",
        "compactions_in_window": n_compact,
        "kv_gbps": round(kv_gbps, 1),
        "hbm_frac": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "compression_ratio": round(cr, 3),
        "retained_per_unit": round(retained / w.units, 1),
        "breakdown": {
            "steps": n_break, "reserve_us": round(res_ms * 1e3, 2),
            "decode_attn_us": round(dec_ev_ms * 1e3, 2), "compact_us": round(cmp_ms * 1e3, 2),
            "compactions": len(t_compact),
            "step_us": round((res_ms + dec_ev_ms + cmp_ms / every) * 1e3, 2),
            "events": "one before and after every call (each adds a few microseconds)",
        },
        "memory": {
            "peak_pages_in_use": peak_pages, "page_bytes": 64 * w.head_dim * 2 * elem,
            "peak_tokens_in_memory": peak_slots, "dense_tokens": dense_tokens,
            "dense_over_peak": round(dense_tokens / peak_slots, 3),
            "per": "one replica (one attention layer, all sequences and KV heads), just before "
                   "its compaction",
        },
        "dead_slot_overhead": round(bytes_read / bytes_alg - 1.0, 5),
        "roofline": {
            "bound": "hbm",
            "kernel": f"k_decode_mfma<{w.head_dim}>",
            "achieved": round(kv_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kv_gbps / HBM_PEAK_GBPS, 4),
            # the counters were taken on the default workload
            "traffic": None if over or args.workload != DEFAULT_WORKLOAD else traffic_from_profile(bytes_alg),
            "algorithmic_bytes_per_launch": int(bytes_alg),
            "launch_us": round(dec_ms * 1e3, 2),
            "launch_time_from": (
                f"two HIP events around {n_launch} back-to-back dms_decode_attn_fill launches "
                "rotating over the replicas (each serving its reserved token again)"
                if launch_ms is not None else
                "HIP events around each dms_decode_attn call of the breakdown pass"),
        },
    }
    log(f"[bench] {tokens_s:.0f} tok/s, {ms_step * 1e3:.1f} us/step ({n_compact} compactions in the "
        f"window), decode {dec_ms * 1e3:.1f} us "
        f"= {kv_gbps:.0f} GB/s ({100 * kv_gbps / HBM_PEAK_GBPS:.1f}% of HBM peak)")
    # context, not a ceiling: what two torch kernels reach on this GPU over 4 GiB (beyond
    # the MALL), a full read (sum) and a device copy (read + write); torch's reduction does
    # not stream at the HBM rate, so the decode kernel can exceed it
    with marked("calibration"):
        cal = calibrate(4.0)
    result["torch_sum_read_gbps"] = cal["sum_read_gbps"]
    result["torch_copy_gbps"] = cal["copy_read_plus_write_gbps"]
    result["kv_frac_of_torch_copy"] = round(kv_gbps / cal["copy_read_plus_write_gbps"], 4)
    if not args.no_chunk:
        with marked("chunk queries"):
            result["chunk"] = chunk_leg(caches, w, dev)
        log(f"[bench] chunk of {result['chunk']['n_query']} queries: {result['chunk']['attn_us']:.1f} us, "
            f"{result['chunk']['tokens_per_s']:.0f} tok/s")
    del inputs, caches, outs
    torch.cuda.empty_cache()
    if not args.no_share:
        with marked("shared prefix"):
            result["shared_prefix"] = shared_prefix_leg(w, dev)
        sp = result["shared_prefix"]
        log(f"[bench] shared prompts: {sp['pages_shared']} pages vs {sp['pages_copied']}, decode "
            f"{sp['decode_us_shared']:.1f} us vs {sp['decode_us_copied']:.1f} us")
        torch.cuda.empty_cache()
    if not args.no_configs:
        result["decode_configs"] = {}
        for n in DECODE_CONFIGS:
            with marked(f"decode {n}"):
                rec = decode_config_leg(n)
            result["decode_configs"][n] = rec
            log(f"[bench] {n}: {rec['ms_per_step'] * 1e3:.1f} us/step, decode {rec['decode_attn_us']:.1f} us "
                f"= {rec['kv_gbps']:.0f} GB/s ({100 * rec['hbm_frac']:.1f}% of HBM peak)")
    if not args.no_prefill:
        log("[bench] masked prefill, 8192 tokens")
        with marked("prefill 8k"):
            result["prefill"] = prefill_leg()
        log(f"[bench] prefill {result['prefill']['ms']:.3f} ms = "
            f"{result['prefill']['roofline']['achieved']:.0f} TFLOP/s causal; gathered "
            f"{result['prefill']['gathered']['ms']:.3f} ms")
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle's masked prefill on a 1024-row sample")
            result["prefill"]["cpu_baseline"] = prefill_cpu_baseline(threads=1)
        torch.cuda.empty_cache()
        log("[bench] masked prefill, head_dim 64 (Llama-3.2-1B-shaped heads), 4096 tokens")
        with marked("prefill 4k head_dim 64"):
            result["prefill_head_dim_64"] = prefill_leg("prefill_4k_d64", relaxed=False)
        torch.cuda.empty_cache()
        with marked("prefill 8k float32"):
            result["prefill_f32"] = prefill_f32_leg()
        log(f"[bench] float32 prefill {result['prefill_f32']['ms']:.2f} ms = "
            f"{result['prefill_f32']['roofline']['achieved']:.0f} TFLOP/s causal")
        torch.cuda.empty_cache()
        with marked("chunked prefill"):
            result["chunked_prefill"] = chunked_prefill_leg()
        log(f"[bench] chunked prefill: last {result['chunked_prefill']['chunk']} tokens in "
            f"{result['chunked_prefill']['ms']:.3f} ms")
        with marked("chunked prefill one sequence"):
            result["chunked_prefill_one_sequence"] = chunked_prefill_leg(batch=1)
        log(f"[bench] chunked prefill, one sequence: "
            f"{result['chunked_prefill_one_sequence']['ms']:.3f} ms split, "
            f"{result['chunked_prefill_one_sequence']['ms_without_split']:.3f} ms without")
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        # the oracle as it stands: BLAS on every core this process may use, then on one;
        # the faster run is the baseline, both are listed
        cores = len(os.sched_getaffinity(0))
        log(f"[bench] timing the oracle on the host (~{2 * args.cpu_seconds:.0f} s: {cores} cores, then 1)")
        runs = [cpu_baseline(w, args.cpu_seconds, threads=cores),
                cpu_baseline(w, args.cpu_seconds, threads=1)]
        result["cpu_baseline"] = max(runs, key=lambda r: r["value"])
        result["cpu_baseline_runs"] = [{k: r[k] for k in ("cores", "value", "seconds_per_step", "kv_gbps")}
                                       for r in runs]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
