"""Host-side checks of bench.py's measurement bookkeeping (no GPU).

The bench line's roofline.traffic comes from a rocprofv3 summary in
profiles/, keyed to a hash of the product kernels' code; these tests pin that
the lookup returns the figure only for the code it was measured on, that the
hash ignores comments and whitespace, and that the committed summaries of the
default (tall Gram) set, the Llama-shaped, MoE and NanoChat sets match the
code as it stands.
"""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

HASHED = ("ns_gemm.hip", "muon_kernels.h", "muon_host.cpp")


def _copy_tree(tmp_path):
    """A minimal copy of the repository layout that bench reads."""
    csrc = tmp_path / "newton_schulz_matrix_momentum_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in HASHED:
        shutil.copy(os.path.join(ROOT, "newton_schulz_matrix_momentum_amd", "csrc", name), csrc / name)
    (tmp_path / "profiles").mkdir()
    return csrc


def _write_profile(tmp_path, workload, sha, nbytes):
    (tmp_path / "profiles" / ("%s_ns_gemm_traffic.md" % workload)).write_text(
        "# traffic\n\n- workload: `%s`\n- kernel_code_sha256: `%s`\n- hbm_bytes_per_launch: `%d`\n"
        % (workload, sha, nbytes))


@pytest.mark.parametrize("workload", ["gram_tall_32x4096x16384", "llama430m_24l_d1024", "moe_64e_d2048",
                                      "nanochat_6l_d192"])
def test_committed_traffic_profiles_match_current_code(workload):
    traffic = bench.recorded_traffic(workload)
    assert traffic is not None and traffic > 0, (
        "profiles/%s_ns_gemm_traffic.md was measured on other product-kernel code; "
        "re-take FETCH_SIZE / WRITE_SIZE" % workload)


def test_traffic_lookup_follows_the_code_hash(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_hash()
    _write_profile(tmp_path, "w_ok", sha, 1234)
    _write_profile(tmp_path, "w_stale", "0" * 64, 5678)
    assert bench.recorded_traffic("w_ok") == 1234.0
    assert bench.recorded_traffic("w_stale") is None
    assert bench.recorded_traffic("w_missing") is None


def test_code_hash_ignores_comments_and_whitespace_only(tmp_path, monkeypatch):
    csrc = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    path = csrc / "ns_gemm.hip"
    src = path.read_text()
    path.write_text("// a new comment line\n/* and a block\n   comment */\n" + src.replace("\n", "\n\n", 5))
    assert bench.kernel_source_hash() == base
    path.write_text(src + "\nconstexpr int kProbe = 1;\n")
    assert bench.kernel_source_hash() != base
