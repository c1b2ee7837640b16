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


def test_mfma_summary_is_read_only_for_the_current_projection_sources(tmp_path, monkeypatch):
    for f in profsum.PROJ_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(profsum.ROOT, f), dst)
    monkeypatch.setattr(profsum, "ROOT", str(tmp_path))
    csv_path = tmp_path / "c.csv"
    csv_path.write_text(
        '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n'
        '1,"isd::(anonymous namespace)::lora_kernel(isd::ProjLaunch)","SQ_INSTS_VALU_MFMA_MOPS_BF16",1000000,0,10000\n'
        '1,"isd::(anonymous namespace)::lora_kernel(isd::ProjLaunch)","SQ_VALU_MFMA_BUSY_CYCLES",2457600,0,10000\n')
    out = tmp_path / "m.txt"
    profsum.mfma(str(csv_path), str(out), "cmd")
    got = profsum.read_mfma(str(out), ("lora_kernel",))
    assert got["lora_kernel"]["gflop"] == 0.512 and got["lora_kernel"]["dur_us"] == 10.0
    assert abs(got["lora_kernel"]["mfma_busy"] - 0.1) < 1e-9        # 2457600 / (1024 x 10 us x 2.4 GHz)
    g = tmp_path / "csrc" / "gemm.hip"
    g.write_text(g.read_text() + "\nnamespace isd { int probe = 1; }\n")
    assert profsum.read_mfma(str(out), ("lora_kernel",)) is None


def test_stall_summary_shares(tmp_path):
    """Wave-cycle shares are the counters' ratios; passes are merged per kernel; busy and
    stall shares are over the dispatch's own duration (10 us here)."""
    k = '"isd::(anonymous namespace)::lora_kernel(isd::ProjLaunch)"'
    head = '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n'
    p1, p2 = tmp_path / "p1.csv", tmp_path / "p2.csv"
    p1.write_text(head + f"1,{k},SQ_WAVE_CYCLES,1000,0,10000\n1,{k},SQ_WAIT_ANY,250,0,10000\n"
                  f"1,{k},SQ_WAIT_INST_ANY,500,0,10000\n1,{k},SQ_ACTIVE_INST_ANY,250,0,10000\n")
    p2.write_text(head + f"1,{k},SQ_VALU_MFMA_BUSY_CYCLES,4915200,0,10000\n"
                  f"1,{k},TCP_PENDING_STALL_CYCLES,3072000,0,10000\n")
    out = tmp_path / "s.txt"
    profsum.stalls(str(out), str(p1), "cmd1", str(p2), "cmd2")
    rows = {l[:34].strip(): l[34:].split() for l in out.read_text().splitlines() if len(l) > 34}
    assert rows["% wave cycles waiting (any)"] == ["25.0"]
    assert rows["% wave cycles waiting to issue"] == ["50.0"]
    assert rows["% MFMA pipes busy"] == ["20.0"]                 # 4915200 / (1024 x 10 us x 2.4 GHz)
    assert rows["% L1 stalled on pending L2 data"] == ["50.0"]   # 3072000 / (256 x 10 us x 2.4 GHz)
    assert "pass 2 command: cmd2" in out.read_text()
