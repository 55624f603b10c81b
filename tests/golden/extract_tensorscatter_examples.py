"""Write tensorscatter_examples.json from the text of the TensorScatter operator page.

The ONNX operator page "TensorScatter" (ai.onnx, since version 24) prints three
worked examples in its Examples section: test_cc_tensorscatter (linear, 4-D),
test_cc_tensorscatter_3d (default attributes, 3-D, two new rows) and
test_cc_tensorscatter_circular (circular, one batch entry wraps). This script
parses the printed inputs and outputs out of the page text, so the stored
values are the page's own, and writes them as JSON next to this file.

Usage: python tests/golden/extract_tensorscatter_examples.py PAGE_TEXT_FILE
where PAGE_TEXT_FILE is a plain-text copy of that page (its Examples section
must be present).
"""
from __future__ import annotations

import ast
import json
import os
import re
import sys

NAMES = ["test_cc_tensorscatter", "test_cc_tensorscatter_3d", "test_cc_tensorscatter_circular"]


def _bracket_block(text: str, start: int) -> tuple[str, int]:
    """Return the balanced [...] block that begins at text[start]."""
    assert text[start] == "["
    depth = 0
    for i in range(start, len(text)):
        if text[i] == "[":
            depth += 1
        elif text[i] == "]":
            depth -= 1
            if depth == 0:
                return text[start:i + 1], i + 1
    raise ValueError("unbalanced brackets")


def _tensor(section: str, name: str) -> dict:
    m = re.search(re.escape(name) + r": shape=\(([^)]*)\), dtype=(\w+)\s*", section)
    if not m:
        raise ValueError(f"{name} not found")
    shape = [int(x) for x in m.group(1).replace(" ", "").split(",") if x]
    values, _ = _bracket_block(section, m.end())
    data = ast.literal_eval(values)
    return {"shape": shape, "dtype": m.group(2), "values": data}


def parse(page_text: str) -> list[dict]:
    line = next(ln for ln in page_text.splitlines() if "test_cc_tensorscatter_circular" in ln)
    out = []
    for k, name in enumerate(NAMES):
        head = line.index(f"**{name}**")
        tail = line.index(f"**{NAMES[k + 1]}**") if k + 1 < len(NAMES) else len(line)
        sec = line[head:tail]
        mode = re.search(r'mode = "(\w+)"', sec)
        axis = re.search(r"axis = (-?\d+)", sec)
        out.append({
            "name": name,
            "citation": "ONNX operator page 'TensorScatter' (ai.onnx, since version 24), "
                        f"Examples section, example {name}",
            "mode": mode.group(1) if mode else "linear",
            "axis": int(axis.group(1)) if axis else -2,
            "past_cache": _tensor(sec, "past_cache"),
            "update": _tensor(sec, "update"),
            "write_indices": _tensor(sec, "write_indices"),
            "present_cache": _tensor(sec, "present_cache"),
        })
    return out


def main() -> None:
    if len(sys.argv) != 2:
        sys.exit("usage: extract_tensorscatter_examples.py PAGE_TEXT_FILE")
    src = sys.argv[1]
    with open(src, encoding="utf-8") as f:
        examples = parse(f.read())
    dst = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tensorscatter_examples.json")
    with open(dst, "w", encoding="utf-8") as f:
        json.dump({"source": "ONNX operator page 'TensorScatter', Examples section",
                   "examples": examples}, f, indent=1)
        f.write("\n")
    print(f"wrote {len(examples)} examples to {dst}")


if __name__ == "__main__":
    main()
