"""Host-side pieces of bench.py: the one-GPU refusal, the byte and tile counts
its rooflines divide by, the code hash that keys the committed counter
summaries, and the shape of the oracle baseline record.  No GPU needed."""

import os
import subprocess
import sys

import torch

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_prefill_algorithmic_bytes_by_hand():
    # B=4, S=8192, 32 query / 8 KV heads, D=128: Q in (268.4 MB), K and V in
    # (2 x 67.1 MB), logits in (1.05 MB), fp32 output out (536.9 MB)
    b, s, hq, hkv, d = 4, 8192, 32, 8, 128
    kv_one = b * s * hkv * d * 2
    expect = b * s * hq * d * 2 + 2 * kv_one + b * s * hkv * 4 + b * s * hq * d * 4
    assert bench.prefill_algorithmic_bytes(b, s, hq, hkv, d) == expect == 940572672
    # the design's own workspace round trip: packed tiles, zeroed far copy and masks, out and in
    assert bench.prefill_workspace_traffic(b, s, hkv, d) == 2 * (2 * 2 * kv_one + b * s * hkv * 4)


def test_prefill_oracle_baseline_record(monkeypatch):
    """The prefill baseline record on a small stand-in workload (same code path)."""
    import dataclasses
    small = dataclasses.replace(wl.get("prefill_8k"), batch=1, context=1024, kv_heads=2)
    monkeypatch.setattr(wl, "get", lambda name: small)
    rec = bench.prefill_cpu_baseline("prefill_8k", threads=1)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "query positions/s"
    assert rec["value"] > 0 and "sample" in rec and rec["seconds_per_call_extrapolated"] > 0


def _tiles_brute(keep, s_len, window, block=32, tile=32):
    """Per unit and query block: gathered tiles holding the kept keys at
    positions <= last query - w, plus every 32-key tile that meets the band
    (first query - w, last query]."""
    b_n, _, h_n = keep.shape
    total = 0
    for bi in range(b_n):
        for h in range(h_n):
            for q0 in range(0, s_len, block):
                i_max = min(s_len, q0 + block) - 1
                kept = sum(int(keep[bi, j, h]) for j in range(0, max(0, i_max - window + 1)))
                gathered = -(-kept // tile)
                band = {j // tile for j in range(max(0, q0 - window + 1), i_max + 1)}
                total += gathered + len(band)
    return total


def test_gathered_tile_count_matches_brute_force():
    gen = torch.Generator().manual_seed(3)
    for s_len, window, rate in [(200, 16, 0.5), (97, 1, 0.9), (64, 40, 0.2), (33, 16, 1.0)]:
        keep = (torch.rand((2, s_len, 3), generator=gen) >= rate).to(torch.int64)
        assert bench.gathered_tiles(keep, s_len, window) == _tiles_brute(keep, s_len, window)


def test_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    b = tmp_path / "b.hip"
    b.write_text("// header\nint f(int x) {\n    return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.src_hash(str(a)) == bench.src_hash(str(b))
    assert bench.src_hash(str(a)) != bench.src_hash(str(c))


def test_oracle_baseline_record():
    w = wl.get("tiny_f32")
    rec = bench.cpu_baseline(w, seconds=0.3, threads=1)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["cores"] == 1
    assert rec["value"] > 0 and rec["seconds_per_step"] > 0 and "sample" in rec


def test_workload_overrides():
    """--batch/--context/--evict-rate/--window/--compact-every/--seed replace the
    workload's fields; a fixed rate replaces a per-unit draw; bad values exit."""
    import argparse

    base = wl.get("qwen32b_width")
    none = argparse.Namespace(**{f: None for f, *_ in bench.OVERRIDES})
    w, over = bench.apply_overrides(base, none)
    assert w is base and over == {}
    args = argparse.Namespace(batch=2, context=1000, evict_rate=0.5, window=8, compact_every=4, seed=9)
    w, over = bench.apply_overrides(base, args)
    assert (w.batch, w.context, w.evict_rate, w.window, w.compact_every, w.seed) == (2, 1000, 0.5, 8, 4, 9)
    assert w.beta_rate is None and over["beta_rate"] is None
    assert (w.kv_heads, w.group, w.head_dim) == (base.kv_heads, base.group, base.head_dim)
    for bad in (dict(batch=0), dict(evict_rate=1.0), dict(window=0)):
        a = argparse.Namespace(**{**vars(none), **bad})
        try:
            bench.apply_overrides(base, a)
        except SystemExit:
            continue
        raise AssertionError(f"{bad} accepted")
