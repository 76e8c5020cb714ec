"""The committed rocprofv3 records that bench.py reads (CPU).

bench.py reports the HBM traffic of the dominant attention kernel from the
FETCH_SIZE / WRITE_SIZE record under profiles/, and only while that record's
SHA-256 matches the kernel source; a kernel change without new counters makes
the field null.  This checks that the committed record belongs to the
committed source and that bench.py finds it."""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _records():
    out = {}
    for line in open(bench.TRAFFIC_RECORD).read().splitlines():
        if line.startswith("traffic-record:"):
            f = dict(kv.split("=", 1) for kv in line.split()[1:])
            out[f["op"]] = f
    return out


def test_traffic_record_matches_the_attention_source():
    sha = hashlib.sha256(open(bench.KERNEL_SOURCE, "rb").read()).hexdigest()
    rec = _records()
    assert set(rec) == {"csa_sparse_attn_prefill", "hca_attn"}
    for op, f in rec.items():
        assert f["sha256"] == sha, f"{op}: record taken on another version of the kernel source"
        assert float(f["bytes"]) > 0
        assert bench.recorded_traffic(op) == float(f["bytes"])


def test_profile_summaries_name_their_commands():
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(pdir))
    assert names, "no profile summaries"
    for n in names:
        assert n.endswith((".md", ".txt")), n
        text = open(os.path.join(pdir, n)).read()
        assert "rocprofv3" in text, f"{n} does not give the command that made it"
        assert len(text) < 64 * 1024, f"{n} is not a short summary"
