"""Host-side logic of bench.py (CPU only): the refusal of more than one GPU,
the algorithmic bytes behind the headline roofline, and the rule that the
committed HBM-traffic profile counts only while the decode sources it was taken
on are unchanged."""

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

import bench
import workloads.generate as generate

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _headline_shape(monkeypatch):
    """The LLaMA-shaped decode layer's sizes and lengths, without its pools."""
    monkeypatch.setattr(generate, "make_decode_case", lambda **kw: SimpleNamespace(**kw))
    kw = generate.decode_llama2_7b_layer()
    return SimpleNamespace(seq_lens=np.asarray(kw.seq_lens), num_seqs=len(kw.seq_lens),
                           num_q_heads=kw.num_q_heads, num_kv_heads=kw.num_kv_heads,
                           head_dim=kw.head_dim, block_size=kw.block_size)


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_headline_algorithmic_bytes(monkeypatch):
    c = _headline_shape(monkeypatch)
    assert c.num_seqs == 64 and c.num_kv_heads == 32 and c.head_dim == 128
    lens = c.seq_lens.astype(np.int64)
    assert (lens >= 512).all() and (lens <= 4096).all()
    kv, total = bench.DecodeRun.algorithmic_bytes(SimpleNamespace(c=c))
    # K and V of every live token, fp16: 512 KiB per token over the 32 layers of
    # the model, 16 KiB per token for this one layer
    assert kv == int(lens.sum()) * 16 * 1024
    blocks = int(((lens + 15) // 16).sum())
    q_and_out = 2 * c.num_seqs * c.num_q_heads * c.head_dim * 2
    assert total == kv + q_and_out + 4 * blocks
    # the figure the committed traffic profile compares its HBM bytes with
    with open(bench.PROFILE_TRAFFIC) as f:
        prof = json.load(f)
    assert prof["algorithmic_bytes_per_launch"] == total


def test_traffic_profile_keyed_to_decode_sources(monkeypatch):
    with open(bench.PROFILE_TRAFFIC) as f:
        prof = json.load(f)
    monkeypatch.setattr(bench, "_decode_sources_sha256", lambda: "0" * 64)
    assert bench._traffic_if_current() is None
    monkeypatch.setattr(bench, "_decode_sources_sha256", lambda: prof["decode_sources_sha256"])
    assert bench._traffic_if_current() == prof["hbm_bytes_per_launch"]
    # the profile's HBM bytes are its calibrated counter readings (the KiB
    # figures are printed to 0.1 KiB)
    cal = prof["copy_calibration"]
    for kind in ("fetch", "write"):
        scale = cal[f"{kind}_scale"]
        got = prof[f"hbm_{kind}_bytes_per_launch"]
        assert abs(got - prof[f"{kind}_size_kib_per_launch"] * 1024 * scale) <= 0.05 * 1024 * scale + 1
    parts = prof["hbm_fetch_bytes_per_launch"] + prof["hbm_write_bytes_per_launch"]
    assert abs(prof["hbm_bytes_per_launch"] - parts) <= 1   # each figure truncated on its own
