"""Readers for the hand-derived fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def _num(tok):
    return float.fromhex(tok) if "0x" in tok else float(tok)


def e2m1_table():
    return {int(a): float(b) for a, b in (l.split() for l in _lines("e2m1_table.txt"))}


def e2m1_rounding():
    return [(float(a), int(b)) for a, b in (l.split() for l in _lines("e2m1_rounding.txt"))]


def mx_blocks():
    blocks, cur = [], None
    for l in _lines("mx_blocks.txt"):
        tag, *rest = l.split()
        if tag == "block":
            cur = {"name": rest[0]}
            blocks.append(cur)
        elif tag == "x":
            cur["x"] = np.array([_num(t) for t in rest])
        elif tag == "byte":
            cur["byte"] = int(rest[0])
        elif tag == "codes":
            cur["codes"] = np.array([int(t) for t in rest], dtype=np.uint8)
    return blocks


def _sparse(tokens, n=256):
    v = np.zeros(n)
    for t in tokens:
        i, x = t.split(":")
        v[int(i)] = float(x)
    return v


def _rle(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out += [int(v)] * int(n)
        else:
            out.append(int(t))
    return np.array(out, dtype=np.uint8)


def slot_cases():
    cases, cur = [], None
    for l in _lines("slot_onehot.txt"):
        tag, *rest = l.split()
        if tag == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif tag in ("key", "value"):
            cur[tag] = _sparse(rest)
        elif tag == "bytes":
            cur["bytes"] = _rle(rest)
    return cases


def decode_two_token():
    d = {"key": {}, "value": {}, "out": {}}
    for l in _lines("decode_two_token.txt"):
        tag, *rest = l.split()
        if tag in ("key", "value"):
            d[tag][int(rest[0])] = _sparse(rest[1:])
        elif tag == "query":
            d["query"] = _sparse(rest)
        elif tag == "out":
            d["out"][int(rest[0])] = float(rest[1])
        elif tag == "scale":
            d["scale"] = float(rest[0])
        elif tag == "seq_len":
            d["seq_len"] = int(rest[0])
    return d


def cache_digests():
    """{workload: (cache bytes, sha256)} from cache_digests.txt (written by
    make_cache_digests.py from the oracle and the seeded inputs only)."""
    out = {}
    for l in _lines("cache_digests.txt"):
        name, nbytes, digest = l.split()
        out[name] = (int(nbytes), digest)
    return out
