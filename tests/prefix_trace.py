"""Runs the hand-derived prefix-cache trace against any allocator with the
oracle's interface (the oracle itself, or an adapter over libpkv)."""

import json
import os

from oracle.allocator import ERR_INVALID, ERR_NO_BLOCKS, AllocatorError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefix_cache_trace.json")
ERRORS = {"no_blocks": ERR_NO_BLOCKS, "invalid": ERR_INVALID}


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def run(make, trace=None):
    """``make(num_blocks, block_size, free_order)`` builds the allocator under test.
    Returns a list of failure descriptions (empty when every expectation holds)."""
    t = trace or load()
    a = make(t["num_blocks"], t["block_size"], t["free_order"])
    rows, fails = {}, []
    for i, op in enumerate(t["ops"]):
        kind = op["op"]
        try:
            if kind == "match":
                got = a.match(op["tokens"], op["cap"])
                if got != op["expect"]:
                    fails.append(f"{i} match {got} != {op['expect']}")
                if "into" in op:
                    rows[op["into"]] = list(got)
            elif kind == "reserve":
                row = rows.setdefault(op["seq"], [])
                slots, _ = a.reserve(row, op["cur_len"], op["n_new"])
                if "expect_error" in op:
                    fails.append(f"{i} reserve should fail")
                elif row != op["expect_row"] or list(slots) != op["expect_slots"]:
                    fails.append(f"{i} reserve row {row} slots {list(slots)}")
            elif kind == "register":
                row = op["rows"] if "rows" in op else rows[op["seq"]]
                n = a.register(op["tokens"], row, op["n_blocks"])
                if "expect_error" in op:
                    fails.append(f"{i} register should fail")
                elif n != op["expect_new"]:
                    fails.append(f"{i} register {n} != {op['expect_new']}")
            elif kind == "release":
                a.release(rows[op["seq"]], len(rows[op["seq"]]))
            elif kind == "check":
                if a.free_list() != op["free"]:
                    fails.append(f"{i} free {a.free_list()} != {op['free']}")
                if a.lru_order() != op["lru"]:
                    fails.append(f"{i} lru {a.lru_order()} != {op['lru']}")
                if a.cached() != op["cached"]:
                    fails.append(f"{i} cached {a.cached()} != {op['cached']}")
                for b, r in op["refs"].items():
                    if a.refcount(int(b)) != r:
                        fails.append(f"{i} ref[{b}] {a.refcount(int(b))} != {r}")
        except AllocatorError as e:
            if ERRORS.get(op.get("expect_error")) != e.code:
                fails.append(f"{i} {kind} raised {e.code}: {e}")
    return fails
