"""Host-side pieces of bench.py: the counter-summary readers that fill
roofline.traffic and roofline.mfma_busy_counters (no GPU)."""
import glob
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, digest, **fields):
    with open(path, "w") as f:
        f.write("# summary\n\n```\nrocprofv3 ...\n```\n\n")
        f.write(f"- kernel_source_sha256: {digest}\n")
        for k, v in fields.items():
            f.write(f"- {k}: {v}\n")


def test_summary_digest_gates_the_values(bench, tmp_path):
    p = tmp_path / "s.md"
    _write(p, "ab" * 32, mfma_busy_frac="0.4279", clock_ghz="2.163")
    kv, src = bench.read_summary(str(p), "ab" * 32)
    assert kv["mfma_busy_frac"] == "0.4279" and kv["clock_ghz"] == "2.163"
    kv, why = bench.read_summary(str(p), "cd" * 32)
    assert kv is None and "changed" in why
    kv, why = bench.read_summary(str(tmp_path / "missing.md"), "ab" * 32)
    assert kv is None and "no counter summary" in why


def test_traffic_scales_both_counters(bench, tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    _write(prof / "attention_kernel_wl_hbm.md", "ee" * 32, fetch_kib_per_launch="100.0",
           write_kib_per_launch="10.0", fetch_scale="2.0", write_scale="1.0")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    traffic, src = bench.read_traffic("wl", "ee" * 32)
    assert traffic == (100.0 * 2.0 + 10.0) * 1024
    assert src == os.path.join("profiles", "attention_kernel_wl_hbm.md")
    busy, why = bench.read_mfma_busy("wl", "ee" * 32)
    assert busy is None and "no counter summary" in why
    _write(prof / "attention_kernel_wl_mfma.md", "ee" * 32, mfma_busy_frac="0.5044", clock_ghz="2.001")
    busy, _ = bench.read_mfma_busy("wl", "ee" * 32)
    assert busy["mfma_busy_frac"] == 0.5044 and busy["clock_ghz"] == 2.001
    # a counted clock above the chip's peak voids the figures derived from it
    _write(prof / "attention_kernel_wl_mfma.md", "ee" * 32, mfma_busy_frac="0.0831",
           clock_ghz="4.715", mfma_busy_frac_at_2_4_ghz="0.1633")
    busy, _ = bench.read_mfma_busy("wl", "ee" * 32)
    assert busy["mfma_busy_frac"] is None and busy["clock_ghz"] is None
    assert busy["mfma_busy_frac_at_2_4_ghz"] == 0.1633 and "exceeds" in busy["note"]


def test_committed_counter_summaries_parse(bench):
    """Every committed counter summary carries a digest and the fields its
    reader needs (whether the digest still matches the kernel is the bench's
    business: a stale summary is reported as such, not used)."""
    files = glob.glob(os.path.join(ROOT, "profiles", "attention_kernel_*_hbm.md")) + \
        glob.glob(os.path.join(ROOT, "profiles", "attention_kernel_*_mfma.md"))
    assert files
    for f in files:
        text = open(f).read()
        digest = [ln.split(":", 1)[1].strip() for ln in text.splitlines()
                  if ln.startswith("- kernel_source_sha256:")]
        assert len(digest) == 1 and len(digest[0]) == 64, f
        kv, _ = bench.read_summary(f, digest[0])
        need = ("fetch_kib_per_launch", "write_kib_per_launch", "fetch_scale", "write_scale") \
            if f.endswith("_hbm.md") else ("mfma_busy_frac", "clock_ghz")
        for k in need:
            float(kv[k])
