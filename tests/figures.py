"""Figures stated on the pages (and published generator outputs) that the
oracle tests pin against, read from tests/golden/page_figures.json, where
each entry names its source."""
import json
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")


def page_figure(key):
    with open(_PATH) as f:
        return json.load(f)[key]
