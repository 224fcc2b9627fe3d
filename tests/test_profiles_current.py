"""The committed profile evidence describes the committed kernels.

The bench line's roofline `traffic` comes from the HBM traffic record under
profiles/, which bench.py attaches only while the record's source hash
matches the attention source; this test fails as soon as that source
changes without the record being taken again.  Every summary also names the
command it came from, and that command runs committed files only."""
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_40_amd", "csrc", "attn_bf16.hip")


def test_traffic_record_matches_the_attention_source():
    rec = json.load(open(os.path.join(PROFILES, "traffic_attn_past_gqa32x8_1m.json")))
    assert rec["kernel_source_sha256"] == hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    # both counter runs scaled by the copy calibration, per launch of the kernel
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"] > 0
    assert len(rec["commands"]) == 2 and all("rocprofv3 --pmc" in c for c in rec["commands"])


def test_every_summary_names_a_command_of_committed_files():
    files = [f for f in os.listdir(PROFILES) if f.endswith((".md", ".txt"))]
    assert files
    for f in files:
        text = open(os.path.join(PROFILES, f)).read()
        cmds = re.findall(r"rocprofv3 [^\n`]*", text)
        assert cmds, f"{f} names no rocprofv3 command"
        for c in cmds:
            assert "_work" not in c and "/root/reference" not in c, (f, c)
            assert "bench.py" in c, (f, c)
