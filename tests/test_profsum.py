"""Host logic of the profile summaries: traffic figures are only reported for
the kernel sources they were measured on."""

import json
import os

from block_sparse_video_map_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _summary(tmp_path, **over):
    rec = {"kernel": "attn_bf16_kernel", "workload": "3a", "bytes_per_launch": 123,
           "source_hash": profsum.source_hash()}
    rec.update(over)
    p = tmp_path / "t.md"
    p.write_text("# x\n\n<!-- traffic: " + json.dumps(rec) + " -->\n")
    return str(p)


def test_matching_summary_is_read(tmp_path):
    r = profsum.read_traffic(_summary(tmp_path), "attn_bf16_kernel", "3a")
    assert r["bytes_per_launch"] == 123


def test_stale_or_foreign_summary_is_ignored(tmp_path):
    assert profsum.read_traffic(_summary(tmp_path, source_hash="0" * 16),
                                "attn_bf16_kernel", "3a") is None
    assert profsum.read_traffic(_summary(tmp_path), "attn_bf16_kernel", "5") is None
    assert profsum.read_traffic(str(tmp_path / "missing.md"), "attn_bf16_kernel", "3a") is None


def test_hash_is_per_kernel(tmp_path):
    assert profsum.source_hash("attn_bf16_kernel") != profsum.source_hash("attn_fp8_kernel")
    p = _summary(tmp_path, kernel="attn_fp8_kernel",
                 source_hash=profsum.source_hash("attn_fp8_kernel"))
    assert profsum.read_traffic(p, "attn_fp8_kernel", "3a")["bytes_per_launch"] == 123
    p = _summary(tmp_path, kernel="attn_fp8_kernel")      # bf16 sources' hash
    assert profsum.read_traffic(p, "attn_fp8_kernel", "3a") is None


def test_short_kernel_names():
    assert profsum.short_name("vsa::(anonymous namespace)::scores_kernel(Plan, int)") == \
        "scores_kernel"
    assert profsum.short_name(
        "void vsa::(anonymous namespace)::gather_kernel<unsigned short, 128>(Plan)") == \
        "gather_kernel<unsigned short, 128>"
