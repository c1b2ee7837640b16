"""The profile summaries' source hash (CPU): it follows code changes of the attention
kernel and of its launch struct, and ignores comments and the other kernels' sections of
the shared launch header."""
import os
import shutil

from strided_verify_propose_amd import profsum


def _copy_sources(tmp_path):
    for f in profsum.ATTN_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(profsum.ROOT, f), dst)


def _edit(path, old, new):
    text = path.read_text()
    assert old in text
    path.write_text(text.replace(old, new, 1))


def test_hash_tracks_attention_code_only(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(profsum, "ROOT", str(tmp_path))
    h0 = profsum.attention_source_hash()
    launch = tmp_path / "csrc" / "launch_types.h"
    # another kernel's section of the header: ignored
    _edit(launch, "int M, Dm, V, NMINI;", "int M, Dm, V, NMINI, EXTRA;")
    assert profsum.attention_source_hash() == h0
    # a comment in the attention section: ignored
    _edit(launch, "struct AttnLaunch {", "struct AttnLaunch {  // reworded")
    assert profsum.attention_source_hash() == h0
    # code in the attention section: tracked
    _edit(launch, "  float scale;", "  float scale, scale2;")
    assert profsum.attention_source_hash() != h0


def test_hash_tracks_the_kernel_source(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(profsum, "ROOT", str(tmp_path))
    h0 = profsum.attention_source_hash()
    att = tmp_path / "csrc" / "attention.hip"
    att.write_text(att.read_text() + "\nnamespace isd { int probe_symbol = 1; }\n")
    assert profsum.attention_source_hash() != h0
