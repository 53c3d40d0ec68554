"""Reader of tests/golden/page_figures.txt: the figures the pages print that CPU tests pin against."""
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.txt")


def page_figure(name: str) -> float:
    """The value stored under ``name`` (each line: name, value, citation)."""
    with open(_PATH, encoding="utf-8") as f:
        for line in f:
            parts = line.split(None, 2)
            if len(parts) >= 2 and not line.lstrip().startswith("#") and parts[0] == name:
                return float(parts[1])
    raise KeyError(name)
