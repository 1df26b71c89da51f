"""The committed rocprofv3 summaries under profiles/ describe the sources in
this tree: every source hash a summary records (a whole kernel file, or the
text of one host function) matches the file as it is now.  A kernel changed
after its profile was taken fails here (bench.py then also reports no
traffic figure for it)."""
import glob
import hashlib
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LINE = re.compile(r"^(\w+_source_sha256): ([0-9a-f]{64})\s+\(([^,)]+)(?:, ([^)]*))?\)\s*$")


def function_text(src: str, name: str) -> str:
    """The text of a C++ function from its signature line to the closing
    brace at the start of a line."""
    i = src.index(" " + name + "(")
    i = src.rindex("\n", 0, i) + 1
    return src[i:src.index("\n}\n", i) + 3]


def recorded_hashes():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        for line in open(path):
            m = LINE.match(line.rstrip("\n"))
            if m:
                out.append((os.path.basename(path),) + m.groups())
    return out


def test_every_profile_records_a_source_hash():
    names = {os.path.basename(p) for p in glob.glob(os.path.join(ROOT, "profiles", "*.txt"))}
    assert names, "no profiles"
    assert names == {h[0] for h in recorded_hashes()}


def test_profile_source_hashes_match_the_tree():
    stale = []
    for prof, key, sha, src, what in recorded_hashes():
        data = open(os.path.join(ROOT, src), "rb").read()
        if what and what.startswith("the text of "):
            name = what.split()[3]
            got = hashlib.sha256(function_text(data.decode(), name).encode()).hexdigest()
        else:
            assert not what, f"{prof}: unknown hash scope {what!r}"
            got = hashlib.sha256(data).hexdigest()
        if got != sha:
            stale.append(f"{prof}: {key} of {src} {what or ''}")
    assert not stale, "profiles taken on other sources: " + "; ".join(stale)
