"""The committed rocprofv3 records describe the library as it stands.

Each counter record under profiles/ carries the hash of the library sources it
was taken on (kernels, launchers and the work planner); the bench reports HBM
traffic only from records whose hash matches.  These checks fail when a
source changes without the records being taken again, and when a summary
lacks the command that made it.
"""

import glob
import json
import os

import pytest

from chunked_prefill_mixed_amd import counters

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
WORKLOADS = ("page1_defaults", "budget8192", "long_context", "heavy_mixed")


def test_every_counter_record_matches_the_current_sources():
    records = sorted(glob.glob(os.path.join(PROFILES, "*_counters.json")))
    assert records
    want = counters.library_source_hash()
    for path in records:
        with open(path) as f:
            rec = json.load(f)
        assert rec["library_source_sha"] == want, os.path.basename(path)
        assert rec["command"].startswith("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc")
        assert rec["dispatches"] > 0 and rec["read_bytes_per_launch"] > 0


def test_source_hash_sees_code_not_comments():
    a = "int x = 1;  // one\n/* a block\n   comment */\nint y = 2;\n"
    b = "int x = 1;\n\n// another comment\nint y = 2;   \n"
    c = "int x = 1;\nint y = 3;\n"
    assert counters._code_only(a) == counters._code_only(b)
    assert counters._code_only(a) != counters._code_only(c)


@pytest.mark.parametrize("kernel", ["append_kernel", "decode_kernel", "chunk_kernel",
                                    "merge_kernel"])
@pytest.mark.parametrize("workload", WORKLOADS)
def test_traffic_records_cover_every_kernel_and_workload(kernel, workload):
    # every measured workload launches all four kernels on its sampled steps
    assert counters.traffic_record(kernel, workload, PROFILES) is not None


def test_summaries_name_their_command():
    texts = sorted(glob.glob(os.path.join(PROFILES, "*.txt")))
    assert texts
    for path in texts:
        with open(path) as f:
            first = f.readline()
        assert first.startswith("command: "), os.path.basename(path)
        # the command runs committed files only
        assert "_work" not in first and "/root/reference" not in first, os.path.basename(path)
