"""The host planner's tree, checked against the oracle's schedule on the CPU.

tests/plan_dump.cpp is compiled with g++ (AddressSanitizer and UBSan on)
together with the library's plan.cpp and prints every plan for K = 1..70 and
some larger K (up to 300), in both schedules, for fp32 and for 16-bit
inputs.  Every merge the GPU path will evaluate must be exactly the node the
oracle defines: same two children (as leaf ranges), same position in the
node order, every input used once, stage operands fp64 above stage 1; blocks
hold at most 16 operands, or 32 (64) when at most 32 (64) 16-bit inputs make
the whole combine one stage.
"""

import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "distributed_sgd_gradient_amd", "csrc")


@pytest.fixture(scope="module")
def plan_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_dump")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(ROOT, "tests", "plan_dump.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


@pytest.fixture(scope="module")
def plans(plan_exe):
    out = subprocess.run([plan_exe], check=True, capture_output=True, text=True,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1")).stdout
    return [json.loads(line) for line in out.splitlines()]


def oracle_nodes(K, schedule):
    """node id -> (lo, mid, hi): the node merges leaves [lo, mid) with [mid, hi)."""
    if schedule == 1:
        return {i: (0, i + 1, i + 2) for i in range(K - 1)}
    ranges = {}
    nodes = {}
    nid = 0
    for level in oracle.tree_schedule(K):
        made = []
        for left, right in level:
            lr = [(r[1], r[1] + 1) if r[0] == "leaf" else ranges[r[1]] for r in (left, right)]
            assert lr[0][1] == lr[1][0]
            nodes[nid] = (lr[0][0], lr[0][1], lr[1][1])
            made.append((nid, (lr[0][0], lr[1][1])))
            nid += 1
        ranges.update(made)
    return nodes


def block_limit(stage, dtype, K, schedule=0):
    """Largest block the planner may form: 16 operands, except the single
    tree stage over at most 32 16-bit inputs (32) or at most 64 (64).
    Chains take 16 whatever the dtype."""
    if stage == 0 and dtype != 0 and K <= 64 and schedule == 0:
        return 32 if K <= 32 else 64
    return 16


def plan_nodes(P):
    """Reconstruct the leaf range of every merge the plan evaluates."""
    slot_range = {}
    got = {}
    for si, st in enumerate(P["stages"]):
        for b in st["blocks"]:
            if si == 0:
                assert all(kind == 0 for kind, _ in b["ops"]), "the first stage reads only inputs"
            else:
                assert all(kind in (0, 1) for kind, _ in b["ops"])
                assert any(kind == 1 for kind, _ in b["ops"]), "a later block holds a lower block's result"
            rng = [(i, i + 1) if kind == 0 else slot_range[i] for kind, i in b["ops"]]
            limit = block_limit(si, P["dtype"], P["K"], P["schedule"])
            assert len(rng) == b["nb"] <= limit and b["nbt"] >= b["nb"]
            for i in range(len(rng) - 1):
                assert rng[i][1] == rng[i + 1][0], "block operands must be adjacent leaf ranges"
            for llo, lhi, rhi, node in b["merges"]:
                assert 0 <= llo < lhi < rhi <= len(rng)
                got[node] = (rng[llo][0], rng[lhi][0], rng[rhi - 1][1])
            lo, hi = rng[0][0], rng[-1][1]
            if b["dst"][0] == 1:
                slot_range[b["dst"][1]] = (lo, hi)
            else:
                assert b["root"] == 1 and (lo, hi) == (0, P["K"])
            # leaf operands are exactly the inputs (read where they are, in any stage)
            leafmask = sum(1 << i for i, (kind, idx) in enumerate(b["ops"]) if kind == 0)
            assert leafmask == b["leafmask"]
    return got


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("schedule", [0, 1])
def test_plan_nodes_match_oracle(plans, schedule, dtype):
    checked = 0
    for P in plans:
        if P["schedule"] != schedule or P["dtype"] != dtype:
            continue
        K = P["K"]
        assert plan_nodes(P) == oracle_nodes(K, schedule), f"K={K}"
        assert sum(1 for st in P["stages"] for b in st["blocks"] if b["root"]) == 1
        checked += 1
    assert checked == 79


def test_16bit_blocks_are_larger(plans):
    """In the tree, up to 32 16-bit inputs (fp16 or bf16) finish in one
    stage of one 32-operand block and up to 64 in one 64-operand block;
    beyond that the first stage uses 16-operand blocks.  A chain takes
    blocks of 16 whatever the dtype (the walk's squared norms lose
    double-double precision over a longer chain): the first 16 inputs, then
    the running result and up to 15 more inputs per stage."""
    seen = set()
    for P in plans:
        if P["K"] in (17, 32, 33, 64, 65):
            K, dt, sc = P["K"], P["dtype"], P["schedule"]
            nstages = len(P["stages"])
            blocks = P["stages"][0]["blocks"]
            if sc == 1:
                assert nstages == 1 + -(-(K - 16) // 15), (K, dt, nstages)
                assert all(b["nb"] <= 16 for st in P["stages"] for b in st["blocks"])
            elif dt != 0 and K <= 64:
                assert nstages == 1
                assert len(blocks) == 1 and blocks[0]["nb"] == K and blocks[0]["nbt"] == (32 if K <= 32 else 64)
                assert blocks[0]["leafmask"] == (1 << K) - 1
            else:
                assert nstages == 2, (K, dt, nstages)
                assert all(b["nb"] <= 16 for b in blocks)
            seen.add((K, dt, sc))
    assert len(seen) == 30


def test_tiles_cover_segments_exactly(plans):
    off = [0, 13, 40]
    for P in plans:
        tiles = np.array(P["tiles"])
        assert tiles[0][0] == 0 and tiles[:, 1].sum() == 40
        assert np.all(tiles[1:, 0] == tiles[:-1, 0] + tiles[:-1, 1])   # contiguous
        for start, length, seg, _, _ in tiles:
            assert off[seg] <= start and start + length <= off[seg + 1]   # inside one segment


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        K = int(rng.choice([rng.integers(1, 40), rng.integers(40, 301)]))
        nseg = int(rng.integers(0, 30))
        kind = rng.integers(0, 3)
        if kind == 0:      # small and empty segments
            lengths = rng.integers(0, 50, size=nseg)
        elif kind == 1:    # ragged, spanning several tiles
            lengths = rng.integers(0, 200000, size=nseg)
        else:              # log-uniform, some empty
            lengths = np.floor(np.exp(rng.uniform(0, np.log(3e5), size=nseg))).astype(np.int64)
            lengths[rng.random(nseg) < 0.1] = 0
        shapes.append((K, int(rng.integers(0, 3)), int(rng.integers(0, 2)), np.concatenate([[0], np.cumsum(lengths)])))
    return shapes


def test_random_shapes_tiles_tree_and_workspace(plan_exe):
    """Seeded random shapes (K up to 300, empty and ragged segments, all
    three dtypes, both schedules): tiles partition every segment with aligned bodies,
    the tree is the oracle's, blocks respect their size limits, and the
    workspace regions are disjoint, ordered and 256-byte aligned."""
    shapes = _random_shapes(400, 2024)
    text = "\n".join(f"{K} {dt} {sc} {len(off) - 1} " + " ".join(str(int(x)) for x in off[1:])
                     for K, dt, sc, off in shapes) + "\n"
    out = subprocess.run([plan_exe, "--stdin"], input=text, check=True, capture_output=True, text=True,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1")).stdout.splitlines()
    assert len(out) == len(shapes)
    for (K, dt, sc, off), line in zip(shapes, out):
        P = json.loads(line)
        assert "error" not in P, (K, P)
        N, nseg, T = int(off[-1]), len(off) - 1, P["tile_rows"]
        tiles = P["tiles"]
        # tiles: in order, contiguous, inside their segment, bodies 8-aligned, bounded length
        pos = 0
        for t, (start, length, seg, _, _) in enumerate(tiles):
            assert start == pos and length >= 1 and off[seg] <= start and start + length <= off[seg + 1]
            first_of_seg = start == off[seg]
            assert first_of_seg or start % 8 == 0
            body = -(-start // 8) * 8 if first_of_seg else start
            assert start + length <= body + T
            pos += length
        assert pos == N
        st = P["seg_tile"]
        assert len(st) == nseg + 1 and st[0] == 0 and st[-1] == len(tiles)
        for s in range(nseg):
            assert all(tiles[t][2] == s for t in range(st[s], st[s + 1]))
            # every tile carries its segment's tile range
            assert all(tiles[t][3:] == [st[s], st[s + 1]] for t in range(st[s], st[s + 1]))
            assert (st[s + 1] > st[s]) == (off[s + 1] > off[s])
        # small one-stage combines of one block of at most 32 operands, no
        # empty segment and few partials for every weighted-sum workgroup to
        # read (at most 2^13 per segment), take the walk and weighted sum in
        # one launch
        nbt0 = P["stages"][0]["blocks"][0]["nbt"]
        reads = max([(st[s + 1] - st[s]) * nbt0 * (nbt0 + 1) // 2 for s in range(nseg)] or [0])
        small = (len(P["stages"]) == 1 and len(P["stages"][0]["blocks"]) == 1 and nbt0 <= 32 and N <= 1 << 22
                 and len(tiles) > 0 and all(st[s + 1] > st[s] for s in range(nseg)) and reads <= 1 << 13)
        if small:
            assert T <= 2048  # one weighted-sum workgroup per tile covers it in one vector step
        assert bool(P["fused"]) == small, (K, dt, sc, off[:5])
        # the walk reads tile-group sums where some segment has 128 tiles or more
        assert bool(P["tile_groups"]) == any(st[s + 1] - st[s] >= 128 for s in range(nseg)), (K, dt, sc)
        # the tree (or chain) is the oracle's, with the block size limits
        assert plan_nodes(P) == oracle_nodes(K, sc), (K, dt, sc)
        for si, stg in enumerate(P["stages"]):
            regions = []
            for b in stg["blocks"]:
                assert b["nb"] <= block_limit(si, dt, K, sc) and b["nbt"] in (2, 4, 8, 16, 32, 64) and b["nbt"] >= b["nb"]
                entries = b["nbt"] * (b["nbt"] + 1) // 2
                assert 0 <= b["poff"] and b["poff"] + entries * len(tiles) <= P["partial_doubles"]
                regions.append((b["poff"], b["poff"] + entries * len(tiles)))
            regions.sort()
            assert all(regions[i][1] <= regions[i + 1][0] for i in range(len(regions) - 1))  # a stage's partials disjoint
        # workspace regions: ordered, 256-aligned, each large enough
        ws = P["ws"]
        assert all(x % 256 == 0 for x in ws) and ws == sorted(ws)
        nodes = max(K - 1, 0)
        sizes = [P["nslots"] * N * 8, P["partial_doubles"] * 8, P["nblocks"] * nseg * 64 * 8,
                 P["nblocks"] * nseg * 64 * 8, P["nblocks"] * nseg * 8,
                 nodes * nseg * 2 * 8, nodes * nseg * 3 * 8, P["nblocks"] * nseg * 4, P["partial_doubles"] * 8]
        # every block carries the error bound of its Gram entries: fp64 sums
        # (fp32 inputs, or a stage over fp64 slots), else the fp32 rounding of
        # the 16-bit matrix cores' chunks
        for si, stg in enumerate(P["stages"]):
            for b in stg["blocks"]:
                reads_slot = any(kind == 1 for kind, _ in b["ops"])
                want = 2.0 ** -44 if (dt == 0 or reads_slot) else 2.0 ** -24 * (1 + 2.0 ** -10)
                assert P["gram_err"][b["desc"]] == want, (K, si)
        for r, size in enumerate(sizes):
            assert ws[r] + size <= ws[r + 1], (K, r)
