"""Host logic of bench.py: the algorithmic bytes each kernel is charged, the kernel names read from
the library's variant string, and the gating of the counter-measured traffic on the kernel source."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_kernel_bytes_of_a_one_token_layer():
    # router rows + x; 9 experts' gate/up (codes + scales); 9 experts' down + x read and written
    kb = bench.kernel_bytes(synth.FLASH, 1, 8)
    assert kb == {"router": 2_621_440 + 5_120, "gateup": 9 * 2_088_960, "down": 9 * 1_044_480 + 2 * 5_120}
    assert sum(kb.values()) - 2 * 5_120 - 5_120 == 30_822_400  # the layer's weights and router


def test_kernel_bytes_of_the_four_token_verify_layer():
    kb = bench.kernel_bytes(synth.FLASH, 4, 32)
    assert kb["gateup"] == 33 * 2_088_960 and kb["down"] == 33 * 1_044_480 + 2 * 4 * 5_120
    assert kb["gateup"] + kb["down"] - 2 * 4 * 5_120 + 2_621_440 == 106_024_960


def test_kernel_names_follow_the_variant_string():
    """Names as the demangler prints them: every template argument, defaults included."""
    n = bench.kernel_names("gfx950-3k-gu5x8-dn8x3-graph", 1)
    assert n == {"router": "void moe::k1_router<1, 8, false, false>(moe::K1Args)",
                 "gateup": "void moe::k2_gateup<1, 8, 4, false, false>(moe::K2Args)",
                 "down": "void moe::k3_down<8, 3, 1, 1, false>(moe::K3Args)"}
    n = bench.kernel_names("gfx950-3k-gu5x8-dn8x3-graph-jit-mfma", 2)
    assert n["router"] == "void moe::k1_router<2, 8, true, false>(moe::K1Args)"
    assert n["gateup"] == "void moe::k2_gateup<2, 8, 2, true, false>(moe::K2Args)"
    n = bench.kernel_names("gfx950-3k-gu5x8-dn8x3-graph-flash", 1)
    assert n["gateup"] == "void moe::flash::k2_gateup<1, 8, 4, false, false>(moe::flash::K2Args)"
    assert n["down"] == "void moe::flash::k3_down<8, 3, 1, 1, false>(moe::flash::K3Args)"


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.source_digest(),
           "kernels": {"k": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "t.md"
    f.write_text("text\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k") == 123
    assert bench.measured_traffic("other") is None
    rec["kernel_source_sha256_16"] = "0" * 16
    f.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.measured_traffic("k") is None


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
