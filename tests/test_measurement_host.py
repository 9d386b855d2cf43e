"""Host-side pieces of the measurement tooling (CPU only): the code-only
source hash that ties a committed counter record to the kernel sources it
was taken from, and that the committed records match the current sources
(otherwise bench.py reports their traffic as null)."""
import json
import os

from gated_delta_rule_amd import traffic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_drops_comments_and_blank_space_but_keeps_literals():
    src = ('int a = 1;   // trailing\n'
           '/* block\n   comment */ int  b = 2;\n\n'
           '    const char* s = "x // y /* z */ \\" w";\n'
           "char c = '\"'; char d = '\\''; // end\n")
    assert traffic.code_only(src) == ('int a = 1;\nint b = 2;\n'
                                      'const char* s = "x // y /* z */ \\" w";\n'
                                      "char c = '\"'; char d = '\\'';")
    # a change to code changes the result, a change to a comment does not
    assert traffic.code_only("x = 1; // a") == traffic.code_only("x = 1; // b")
    assert traffic.code_only("x = 1;") != traffic.code_only("x = 2;")


def test_committed_records_match_the_current_sources():
    for kind, name in (("prefill", "chunk_fwd_workload1_traffic.json"),
                       ("prefill", "chunk_fwd_workload1_mfma.json"),
                       ("decode", "decode_step_workload4_traffic.json"),
                       ("backward", "chunk_bwd_workload1_traffic.json")):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        assert rec["kernel_sources_sha256_16"] == traffic.sources_hash(kind), name
