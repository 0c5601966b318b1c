"""Loader for the page-printed layout fixtures in tests/golden/."""
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def tup(x):
    if isinstance(x, list):
        return tuple(tup(v) for v in x)
    return x


def layout_cases():
    with open(os.path.join(HERE, "golden", "layout_pages.json")) as f:
        data = json.load(f)
    return data["cases"]
