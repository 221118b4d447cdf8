"""Host-side logic of bench.py (no GPU): the HBM-traffic record lookup."""
import importlib.util
import json
import os

import pytest

import bench
from exact_attention_77_amd.build import fingerprint
from synth_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def _records():
    if not os.path.exists(RECORD):
        return {}
    return {k: v for k, v in json.load(open(RECORD)).items() if isinstance(v, dict)}


@pytest.mark.parametrize("name", sorted(_records()))
def test_traffic_record_is_found_when_sources_match(name):
    rec = _records()[name]
    current = all(fingerprint(os.path.basename(s)) == f for s, f in rec["fingerprints"].items())
    got = bench.measured_traffic(WORKLOADS[name])
    if current:
        assert got == rec["read_bytes"] + rec["write_bytes"] and got > 0
    else:
        assert got is None


def test_traffic_record_rejected_after_source_change(tmp_path, monkeypatch):
    if not _records():
        pytest.skip("no recorded HBM traffic in this tree")
    name = sorted(_records())[0]
    recs = json.load(open(RECORD))
    src = next(iter(recs[name]["fingerprints"]))
    recs[name]["fingerprints"][src] = "0" * 16          # as if the kernel had changed
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(WORKLOADS[name]) is None


def test_strip_comments_keeps_code_and_literals():
    from exact_attention_77_amd.build import strip_comments
    src = ('int a = 1; // one\n'
           'const char* s = "// kept /* kept */";\n'
           '/* two\n   lines */ char q = \'\\\'\'; char r = \'"\';\n')
    out = strip_comments(src)
    assert "one" not in out and "two" not in out and "lines" not in out
    assert '"// kept /* kept */"' in out and "char q = '\\''" in out and "char r = '\"'" in out
    assert out.count("\n") == src.count("\n")


def test_fingerprint_ignores_comment_edits_only(tmp_path, monkeypatch):
    from exact_attention_77_amd import build
    (tmp_path / "k.hip").write_text("__global__ void k(int* p) { p[0] = 1; }  // a kernel\n")
    monkeypatch.setattr(build, "CSRC", str(tmp_path))
    f0 = build.fingerprint("k.hip")
    (tmp_path / "k.hip").write_text("/* the same kernel */\n__global__ void k(int* p) { p[0] = 1; }\n")
    assert build.fingerprint("k.hip") == f0
    (tmp_path / "k.hip").write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert build.fingerprint("k.hip") != f0


def test_fingerprint_does_not_depend_on_the_tree_location(tmp_path, monkeypatch):
    """The same sources copied elsewhere (as for a run on another machine)
    keep their fingerprint."""
    import importlib
    import shutil
    from exact_attention_77_amd import build
    f0 = build.fingerprint("fwd_bf16.hip")
    copy = tmp_path / "elsewhere" / "exact_attention_77_amd"
    shutil.copytree(os.path.dirname(build.__file__), copy, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    spec = importlib.util.spec_from_file_location("build_copy", copy / "build.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.ROOT != build.ROOT and mod.fingerprint("fwd_bf16.hip") == f0
