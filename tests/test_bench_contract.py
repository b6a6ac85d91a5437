"""Host-side checks of bench.py (no GPU): the one-GPU contract and the use of
the committed rocprofv3 counter summaries for the roofline's traffic field."""
import importlib.util
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 2" in r.stderr and r.stdout.strip() == ""


def test_traffic_is_read_only_while_the_kernel_source_matches(tmp_path, monkeypatch):
    bench = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest(str(src))
    (prof / "k.md").write_text(f"traffic_bytes_per_launch: 1.5e+09\nkernel_source_sha256: {digest}\n")
    assert bench.committed_traffic(str(src), "k.md") == 1.5e9
    src.write_text("// kernel v2\n")  # the source changed after the counters were taken
    assert bench.committed_traffic(str(src), "k.md") is None
    assert bench.committed_traffic(str(src), "missing.md") is None


def test_committed_profiles_are_well_formed():
    # every counter summary under profiles/ names its command, its traffic and the digest of
    # the kernel source it was taken on; bench.py uses the traffic only while that digest
    # matches the current source (otherwise the bench line reports traffic null)
    bench = load_bench()
    checks = {"prefill_ws_long_prefill.md": "prefill_sym.hip", "prefill_ws_jrt_prefix.md": "prefill_sym.hip",
              "prefill_ws_layer_prefill.md": "prefill_sym.hip", "prefill_quad_tiny_f32.md": "prefill_exact.hip",
              "decode_state_passing.md": "decode.hip",
              "decode_compact_state_passing.md": "decode.hip", "swa_prefill_w64.md": "swa.hip",
              "swa_prefill_w128.md": "swa.hip", "swa_decode_w128.md": "swa.hip"}
    csrc = os.path.join(ROOT, "recurrent_lm_sequence_amd", "csrc")
    for prof, src in checks.items():
        text = open(os.path.join(ROOT, "profiles", prof)).read()
        assert "rocprofv3" in text, prof
        assert re.search(r"traffic_bytes_per_launch:\s*[0-9.eE+]+", text), prof
        m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
        assert m, prof
        got = bench.committed_traffic(os.path.join(csrc, src), prof)
        current = m.group(1) == bench.source_digest(os.path.join(csrc, src))
        assert (got is not None) == current, prof
