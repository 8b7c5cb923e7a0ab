"""Readers for the hand-computed fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cases(name):
    case = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                case = {"name": rest.strip(), "rows": [], "y": [], "a": []}
            elif key == "end":
                yield case
                case = None
            else:
                case.setdefault("_lines", []).append((key, rest.split()))
                if key == "row":
                    case["rows"].append(bytes(int(t, 16) for t in rest.split()))
                elif key == "k":
                    case["k"] = int(rest)
                elif key == "x":
                    case["x"] = rest.split()
                elif key in ("y", "a"):
                    case[key].extend(float(t) for t in rest.split())
                elif key == "r":
                    case["r"] = int(rest)


def q4_0_block_cases(fixture="q4_0_blocks.txt", block_bytes=18):
    """Hand-computed Q4_0 cases: dict(name, k, w uint8[n, k/32*18], x float16[k], y, a)
    (Q8_0 cases with fixture q8_0_blocks.txt and 34-byte blocks)."""
    out = []
    for c in _cases(fixture):
        k = c["k"]
        rb = k // 32 * block_bytes
        for r in c["rows"]:
            assert len(r) == rb, (c["name"], len(r), rb)
        w = np.frombuffer(b"".join(c["rows"]), dtype=np.uint8).reshape(len(c["rows"]), rb).copy()
        if c["x"] == ["iota"]:
            x = np.arange(1, k + 1, dtype=np.float64)
        else:
            x = np.array([float(t) for t in c["x"]], dtype=np.float64)
        assert x.size == k, c["name"]
        x16 = x.astype(np.float16)
        assert np.array_equal(x16.astype(np.float64), x), "fixture x must be exact in f16"
        out.append(dict(name=c["name"], k=k, w=w, x=x16, y=np.array(c["y"]), a=np.array(c["a"])))
    return out


def argmax_cases():
    out = []
    for c in _cases("argmax.txt"):
        ys = [v for key, v in c["_lines"] if key == "y"][0]
        out.append(dict(name=c["name"], y=np.array([float(t) for t in ys]), r=c["r"]))
    return out


def rms_norm_cases():
    """Hand-worked final-norm cases: dict(name, h float16[K], g float16[K], eps float32, x float16[K])."""
    out = []
    for c in _cases("rms_norm.txt"):
        f = {key: v for key, v in c["_lines"]}
        h = np.array([float(t) for t in f["h"]], dtype=np.float64)
        g = np.array([float(t) for t in f["g"]], dtype=np.float64)
        x = np.array([float(t) for t in f["x"]], dtype=np.float64)
        eps = float(f["eps"][0])
        for name, v in (("h", h), ("g", g), ("x", x)):
            assert np.array_equal(v.astype(np.float16).astype(np.float64), v), (c["name"], name)
        assert float(np.float32(eps)) == eps, c["name"]
        assert h.size == g.size == x.size, c["name"]
        out.append(dict(name=c["name"], h=h.astype(np.float16), g=g.astype(np.float16), eps=eps,
                        x=x.astype(np.float16)))
    return out


def q8_0_block_cases():
    """Hand-computed Q8_0 cases, as q4_0_block_cases with 34-byte blocks."""
    return q4_0_block_cases("q8_0_blocks.txt", 34)
