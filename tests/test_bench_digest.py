"""bench.py's device-source digest: comment edits leave it unchanged, code edits change it."""
import os
import shutil

import bench

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "mixture_experts_layer_table_amd", "csrc")


def _copy(tmp_path):
    d = tmp_path / "csrc"
    shutil.copytree(CSRC, d)
    return d


def test_comment_edits_keep_the_digest(tmp_path):
    d = _copy(tmp_path)
    base = bench.source_digest(str(d))
    assert base == bench.source_digest()
    p = d / "tiles.h"
    text = p.read_text()
    p.write_text("// a new line comment\n/* a block\n   comment */\n" + text.replace("\n", "  // trailing\n", 3))
    assert bench.source_digest(str(d)) == base


def test_code_edits_change_the_digest(tmp_path):
    d = _copy(tmp_path)
    base = bench.source_digest(str(d))
    p = d / "tiles.h"
    text = p.read_text()
    assert "kTileN = 256" in text
    p.write_text(text.replace("kTileN = 256", "kTileN = 128"))
    assert bench.source_digest(str(d)) != base


BUILD = os.path.join(os.path.dirname(CSRC), "build.py")


def test_host_source_edits_change_the_digest(tmp_path):
    d = _copy(tmp_path)
    base = bench.source_digest(str(d))
    p = d / "plan.cpp"
    text = p.read_text()
    assert "kAlign" in (d / "plan.h").read_text()
    p.write_text(text.replace("q.max_mtiles = q.R / q.tile.BM + q.cap + 1;",
                              "q.max_mtiles = q.R / q.tile.BM + q.cap + 2;"))
    assert bench.source_digest(str(d)) != base


def test_build_flag_edits_change_the_digest(tmp_path):
    b = tmp_path / "build.py"
    text = open(BUILD).read()
    assert '"-O3"' in text
    b.write_text(text)
    base = bench.source_digest(CSRC, str(b))
    assert base == bench.source_digest()
    b.write_text(text.replace('"-O3"', '"-O2"'))
    assert bench.source_digest(CSRC, str(b)) != base
    b.write_text(text.replace('"-O3", ', '"-O3",  # a comment\n    '))
    assert bench.source_digest(CSRC, str(b)) == base
