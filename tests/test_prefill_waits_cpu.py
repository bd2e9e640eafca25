"""The prefill kernel's counted waits, replayed on the CPU from its own source.

The prefill body streams K / V tiles into LDS with loads that complete in issue
order and ends each iteration with ``s_waitcnt vmcnt(N)``: at most N of the wave's
loads may still be in flight. That wait is correct only if every tile the next
iteration reads was issued at least N loads before it. This test reads the issue
order of the item prologue and of the loop body, the loads per call and the wait
counts from ``prefill_item.h`` itself (so a change to the kernel's order changes
what is checked), replays them, and checks:

* the prologue wait leaves K(0), V(0) and K(1) complete (the prologue's scores read
  K(0); iteration 0 reads K(1) and V(0));
* the wait at the end of iteration j leaves K(j+2) and V(j+1) complete (iteration
  j+1 reads them);
for both page modes (one page id per wave and tile, or one per lane token).

The second test applies an earlier prologue order (both page-id fetches before the
first tile load) to the source text and requires the replay to find the tile it
leaves uncovered.
"""

from __future__ import annotations

import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_173_amd", "csrc", "prefill_item.h")


def _const(src, name):
    m = re.search(rf"constexpr int {name} = (\d+);", src)
    assert m, f"{name} not found"
    return int(m.group(1))


def _eval(expr, env):
    expr = expr.strip()
    assert re.fullmatch(r"[\w\s\*\+\-\(\)/]+", expr), expr
    return int(eval(expr, {"__builtins__": {}}, dict(env)))


def model(src: str, uniform: bool):
    """(loads per iteration, prologue events, body events) from the source text.
    Events: ("fetch", tile) / ("k", tile) / ("v", tile) / ("wait", N); body tiles are
    offsets from j."""
    kt = _const(src, "KT")
    nw = int(re.search(r"int RB = 1, int NW = (\d+)>", src).group(1))
    env = {"KT": kt, "NW": nw}
    env["kRpw"] = _eval(re.search(r"constexpr int kRpw = ([^;]+);", src).group(1), env)
    env["kLpw"] = _eval(re.search(r"constexpr int kLpw = ([^;]+);", src).group(1), env)
    m = re.search(r"constexpr int kLoadsPerIter = MODE == kPagedUniform \? ([^:]+) : ([^;]+);",
                  src)
    per_iter = _eval(m.group(1) if uniform else m.group(2), env)
    env["kLoadsPerIter"] = per_iter
    # loads of one call: a tile's K (or V) is kLpw loads; a page-id fetch is the rest
    per_tile = env["kLpw"]
    per_fetch = per_iter - 2 * per_tile
    assert per_fetch >= 1

    def events(block, offset_pat):
        ev = []
        for m in re.finditer(r"fetch_pids\(" + offset_pat + r"\)|"
                             r"issue\(" + offset_pat + r", \w+, (kbase|vbase)|"
                             r"wait_vm<([^>]+)>\(\)", block):
            if m.group(0).startswith("fetch_pids"):
                ev.append(("fetch", int(m.group(1))))
            elif m.group(0).startswith("issue"):
                ev.append(("k" if m.group(3) == "kbase" else "v", int(m.group(2))))
            else:
                ev.append(("wait", _eval(m.group(4), env)))
        return ev

    pro = src[src.index("  if (ntiles > 0) {"):]
    pro = pro[:pro.index("lds_barrier();")]
    prologue = events(pro, r"(\d+)")
    body = src[src.index("  auto body = [&](int j, auto ph"):]
    body = body[:body.index("\n  };\n")]
    # the generic branch spells out the tile offsets (the uniform branch issues
    # the same tiles through group records built from them)
    gen = body[body.index("    } else {"):]
    order = events(body[:body.index("    if constexpr (MODE == kPagedUniform) {")], r"j \+ (\d+)")
    order += [e for e in events(gen, r"j \+ (\d+)") if e[0] in ("k", "v")]
    order += [e for e in events(body, r"j \+ (\d+)") if e[0] == "wait"]
    return per_iter, per_tile, per_fetch, prologue, order


def replay(src: str, uniform: bool, iterations: int = 12):
    """Returns the list of violations: (where, tile, loads issued after it, wait count)."""
    per_iter, per_tile, per_fetch, prologue, body = model(src, uniform)
    issued = []            # (kind, tile) per load, in issue order
    bad = []

    def issue(kind, tile):
        n = per_fetch if kind == "fetch" else per_tile
        issued.extend([(kind, tile)] * n)

    def check(where, need, n_wait):
        for kind, tile in need:
            last = max(i for i, e in enumerate(issued) if e == (kind, tile))
            after = len(issued) - 1 - last
            if after < n_wait:
                bad.append((where, f"{kind.upper()}({tile})", after, n_wait))

    for kind, x in prologue:
        if kind == "wait":
            check("prologue", [("k", 0), ("v", 0), ("k", 1)], x)
        else:
            issue(kind, x)
    assert sum(1 for e in body if e[0] == "wait") == 1
    assert [e for e in body if e[0] != "wait"][-1] != ("wait",)
    for j in range(iterations):
        for kind, x in body:
            if kind == "wait":
                check(f"iteration {j}", [("k", j + 2), ("v", j + 1)], x)
            else:
                issue(kind, j + x)
    return bad, per_iter


@pytest.mark.parametrize("uniform", [True, False], ids=["page-uniform", "generic"])
def test_every_counted_wait_covers_the_next_iterations_tiles(uniform):
    src = open(SRC).read()
    bad, per_iter = replay(src, uniform)
    assert per_iter == (5 if uniform else 6)          # 4 waves: two loads per tile and wave
    assert not bad, bad


def test_the_earlier_prologue_order_is_caught():
    """Both page-id fetches before the first tile load (an order this kernel once had):
    V(1)'s last load then has one load too few after it at iteration 0's wait."""
    src = open(SRC).read()
    new = ("    issue(0, p0, kbase, sK0, true);\n"
           "    issue(0, p0, vbase, sV0, false);\n"
           "    issue(1, p1, kbase, sK1, true);\n"
           "    pid_k0 = fetch_pids(4);\n"
           "    issue(2, p2, kbase, sK2, true);\n"
           "    issue(1, p1, vbase, sV1, false);\n"
           "    pid_k1 = fetch_pids(5);\n")
    old = ("    pid_k0 = fetch_pids(4);\n"
           "    pid_k1 = fetch_pids(5);\n"
           "    issue(0, p0, kbase, sK0, true);\n"
           "    issue(0, p0, vbase, sV0, false);\n"
           "    issue(1, p1, kbase, sK1, true);\n"
           "    issue(2, p2, kbase, sK2, true);\n"
           "    issue(1, p1, vbase, sV1, false);\n")
    assert new in src, "the prologue's issue order changed: update this test"
    for uniform in (True, False):
        bad, _ = replay(src.replace(new, old), uniform)
        assert ("iteration 0", "V(1)", 9 if uniform else 10, 10 if uniform else 12) in bad, bad
