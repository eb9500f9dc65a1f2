"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
roofline divides by, the refusal of more than one GPU, and the guards on
the committed counter summaries."""
import json
import os
import subprocess
import sys

import pytest

import bench
import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def defined_bytes(w):
    # x once, K rows written, K rows read back, the output row, logits,
    # routing metadata (index, weight, slot, source: 4 x 4 B written and
    # read), the node mask, and the per-expert/rank/node arrays
    b = 4 if w.x_dtype == mi.F32 else 2
    return w.T * ((2 * w.K + 2) * w.H * b + 4 * w.E + 32 * w.K + 8) + \
        8 * (w.E + w.R + w.N)


@pytest.mark.parametrize("w", [mi.MIXTRAL, mi.QWEN3, mi.DEEPSEEK_V3,
                               mi.DEEPSEEK_V3_DECODE, mi.KIMI],
                         ids=lambda w: w.name)
def test_algorithmic_bytes(w):
    assert w.algorithmic_bytes() == defined_bytes(w)


def test_deepseek_bytes_per_launch():
    w = mi.DEEPSEEK_V3
    kb = bench.kernel_bytes(w)
    T, H, K = w.T, w.H, w.K
    assert kb["pack"] == T * H * 2 * (1 + K) + 4 * T * K
    assert kb["combine"] == T * K * H * 2 + T * H * 2 + 12 * T * K + 4 * w.E
    # the whole path moves 4249.0 MB per step
    assert abs(w.algorithmic_bytes() / 1e6 - 4249.0) < 0.1


def test_fp8_bytes_per_launch():
    # payload of a row: H one-byte codes and H/128 fp32 scales, not padding
    w = mi.DEEPSEEK_V3
    kb = bench.fp8_kernel_bytes(w, 128)
    T, H, K = w.T, w.H, w.K
    assert kb["pack_fp8"] == T * H * 2 + T * K * (H + 4 * H // 128) + 4 * T * K
    assert kb["combine_fp8"] == T * K * 7392 + T * H * 2 + 12 * T * K + 4 * w.E


def test_alu_peak():
    # 256 CUs x 64 lanes x 2.4 GHz
    assert bench.ALU_PEAK_TOPS == pytest.approx(39.3216)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_summaries_follow_the_sources(tmp_path, monkeypatch):
    # a summary taken from other source text is not reported
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "pack", ["k.hip"])
    entry = {"bytes_per_launch": 123.0,
             "source_sha": bench.source_digest(["k.hip"])}
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"pack/deepseek_v3": entry}))
    assert bench.load_traffic("pack", "deepseek_v3") == 123.0
    assert bench.load_traffic("pack", "kimi") is None
    src.write_text("kernel v2")
    assert bench.load_traffic("pack", "deepseek_v3") is None


def test_decode_rule_matches_the_library():
    # bench.py reports the decode kernel for the batches the library sends
    # to it; the two limits are read from the kernel source
    import re
    src = open(os.path.join(ROOT, "combine_moe_topk_amd", "csrc",
                            "decode.hip")).read()
    t = int(re.search(r"kDecodeMaxTokens = (\d+);", src).group(1))
    tk = int(re.search(r"kDecodeMaxIds = (\d+);", src).group(1))
    assert (bench.DECODE_MAX_T, bench.DECODE_MAX_TK) == (t, tk)


def test_traffic_source_is_labelled(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("kernel v1")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "pack", ["k.hip"])
    assert "profiles/traffic.json" in bench.traffic_source("pack", "kimi", 1.0)
    assert bench.traffic_source("pack", "kimi", None).startswith("none")
