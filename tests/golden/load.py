"""Readers for the cited page fixtures in this directory."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows(name):
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def sum_rows_iota():
    """[(case, count, offset, step)] from the page's eight check cases."""
    return [(c, int(n), float(o), float(s)) for c, n, o, s in _rows("sum_rows_iota.txt")]


def launch_fill():
    """[(element_count, workgroup_size, workgroups)]."""
    return [tuple(int(v) for v in r) for r in _rows("launch_fill.txt")]
