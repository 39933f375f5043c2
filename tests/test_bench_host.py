"""Host-side behaviour of bench.py (no GPU): the one-GPU refusal, the kernel-source hash that
gates counter-derived traffic, and the committed traffic summaries it reads."""
import glob
import os
import subprocess
import sys

import bench
from exact_attention_17_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_code_only_drops_comments_and_whitespace_but_not_strings():
    src = 'int a = 1;  // note\n/* block\n comment */ f("x // y", \'c\');\n'
    assert bench._code_only(src) == 'inta=1;f("x // y",\'c\');'


def test_comment_edits_keep_the_hash(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_attention_17_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "fa_fwd_kernel.h").write_text("int k() { return 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    (csrc / "fa_fwd_kernel.h").write_text("// a comment\nint k() {\n  return 1;  /* same */\n}\n")
    assert bench.kernel_source_hash() == h1
    (csrc / "fa_fwd_kernel.h").write_text("int k() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_traffic_is_read_only_for_the_current_kernel(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_attention_17_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "fa_fwd_kernel.h").write_text("int k() { return 1; }\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    cfg = fa.TileConfig(256, 64, 8, 3, 2)
    tail = "tile: 256,64,8,3,2\nnum_splits: 1\nhbm_bytes_per_launch: 1234\n"
    prof = tmp_path / "profiles" / "fa_fwd_full_traffic.txt"
    prof.write_text("# header: ignored\nworkload: full\nkernel_source_hash: %s\n%s" % (h, tail))
    assert bench.read_traffic("full", cfg, 1) == 1234
    assert bench.read_traffic("varlen", cfg, 1) is None  # no such profile
    assert bench.read_traffic("full", fa.TileConfig(128, 32, 4, 2, 4), 1) is None  # another tile's numbers
    assert bench.read_traffic("full", cfg, 4) is None  # another split count's
    prof.write_text("workload: full\nkernel_source_hash: 0000000000000000\n" + tail)
    assert bench.read_traffic("full", cfg, 1) is None  # taken on other kernel sources
    prof.write_text("workload: gqa\nkernel_source_hash: %s\n%s" % (h, tail))
    assert bench.read_traffic("full", cfg, 1) is None  # another workload's numbers
    # a second tile's summary, named for its tile
    prof.write_text("workload: full\nkernel_source_hash: %s\n%s" % (h, tail))
    alt = tmp_path / "profiles" / "fa_fwd_full_256-96-8-3-2_traffic.txt"
    alt.write_text("workload: full\nkernel_source_hash: %s\ntile: 256,96,8,3,2\nnum_splits: 1\n"
                   "hbm_bytes_per_launch: 999\n" % h)
    assert bench.read_traffic("full", cfg, 1) == 1234
    assert bench.read_traffic("full", fa.TileConfig(256, 96, 8, 3, 2), 1) == 999
    assert bench.read_traffic("full", fa.TileConfig(256, 32, 8, 3, 2), 1) is None


def test_committed_traffic_summaries_are_consistent():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "fa_fwd_*_traffic.txt")))
    assert paths
    for p in paths:
        vals = {}
        with open(p) as f:
            for line in f:
                if line.startswith("#") or ":" not in line:
                    continue
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
        name = os.path.basename(p)[len("fa_fwd_"):-len("_traffic.txt")]
        # fa_fwd_<workload>_traffic.txt, or fa_fwd_<workload>_<tile>_traffic.txt for another tile
        assert name == vals["workload"] or name == vals["workload"] + "_" + vals["tile"].replace(",", "-")
        assert int(vals["hbm_bytes_per_launch"]) == int(vals["fetch_bytes_per_launch"]) + int(
            vals["write_bytes_per_launch"])
        assert len(vals["kernel_source_hash"]) == 16
        assert len(vals["tile"].split(",")) == 5 and int(vals["num_splits"]) >= 1
