"""Load the DequantizePacked page's own Python notation as a second reading.

The page defines decoding twice: in its "Mathematical decoding rules" (which
the oracle restates in C) and in its "Equivalent Python notation".  This
helper extracts the second notation's code blocks from a local text copy of
the page at run time -- nothing of it is stored in this repository -- and
executes them in a private namespace, so tests can compare the oracle with an
independent reading.  The copy's path comes from the NQ_PAGE_TEXT environment
variable; without it (or without the file) load() returns None and the tests
that use it are skipped.  CPU tests only.
"""
import os

PAGE = os.environ.get("NQ_PAGE_TEXT", "")


def _segment(lines, start_pred, end_pred, include_end):
    for i, line in enumerate(lines):
        if start_pred(line):
            for j in range(i + 1, len(lines)):
                if end_pred(lines[j]):
                    return lines[i:j + 1] if include_end else lines[i:j]
    raise ValueError("segment not found")


def load():
    if not PAGE or not os.path.exists(PAGE):
        return None
    with open(PAGE, encoding="utf-8") as f:
        lines = f.read().split("\n")
    # restrict to page 2 (the ONNX page)
    p2 = next(i for i, l in enumerate(lines) if "DequantizePacked decoding specification" in l)
    lines = lines[p2:]
    common = _segment(lines, lambda l: l == "import math",
                      lambda l: l.startswith("Conventional, K-quant"), False)
    block = _segment(lines, lambda l: l.startswith("def decode_block("),
                     lambda l: l.strip() == 'raise ValueError("Unknown format")', True)
    iq = _segment(lines, lambda l: l.startswith("def decode_iq("),
                  lambda l: l == "    return y", True)
    books = _segment(lines, lambda l: l.startswith("CODEBOOKS = {"), lambda l: l == "}", True)
    src = "\n".join(common + [""] + block + [""] + iq + [""] + books) + "\n"
    ns = {}
    exec(compile(src, "<DequantizePacked page: Python notation>", "exec"), ns)
    return ns


def kind_of(fmt):
    """Map an identifier such as 'gguf:q4_k' to the notation's kind 'Q4_K'."""
    assert fmt.startswith("gguf:")
    return fmt[5:].upper()
