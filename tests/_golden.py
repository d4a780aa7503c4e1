"""Reader of the hand-worked prefill page-order example (test helper)."""
import os


def prefill_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "prefill_pages_example.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split("->")
        f = dict(kv.split("=") for kv in lhs.split()[1:])
        ints = lambda v: [int(x) for x in v.split(",")]
        tabs, stack = rhs.split("|")
        tables = {}
        for t in tabs.split():
            s, v = t.split(":")
            tables[int(s)] = [] if v == "-" else ints(v)
        yield ints(f["slots"]), ints(f["lens"]), ints(f["max_new"]), tables, ints(stack.strip())
