"""Host checks of the single-launch planner (csrc/plan.hpp), compiled with
g++ into a small driver: when the decode step runs as one persistent
launch, the whole grid (or the part kept on each XCD) must be resident at
once, since its workgroups wait for each other."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "compensated_kv_selection_amd", "csrc")

SHARE_MAX, CAND_MAX, PAGE_LIMIT = 256, 4608, 1 << 18


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "plan_driver.cpp"),
                    "-o", exe], check=True)

    def run(cases):
        text = "\n".join(" ".join(str(x) for x in c) for c in cases) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]
    return run


def case(n_chunks, kmax, pairs, resident=512, xcds=8, share=None, num_pages=8192, max_rounds=1000):
    share = share if share is not None else max(1, -(-kmax // n_chunks)) if kmax else 1
    return (n_chunks, kmax, share, SHARE_MAX, CAND_MAX, num_pages, PAGE_LIMIT, resident, pairs, xcds, max_rounds)


def rounds_of(n_chunks, n_val, per_round, pairs):
    return -(-pairs // per_round)


def test_headline_shape(driver):
    # 128K tokens = 32 chunks of 256 blocks per (sequence, KV head), 8 pairs,
    # two workgroups per CU on 256 CUs: one round, every pair on its own XCD
    assert driver([case(32, 32, 8)]) == [(1, 32, 8, 8)]
    # without a verified XCD mapping the pairs are spread
    assert driver([case(32, 32, 8, xcds=0)]) == [(1, 32, 8, 0)]


def test_spare_pages_take_fewer_value_workgroups(driver):
    # 33 chunks (a table with room for more pages): 33 + 33 per pair do not
    # fit on one XCD's 64 slots, 33 + 31 do
    assert driver([case(33, 32, 8)]) == [(1, 31, 8, 8)]


@pytest.mark.parametrize("kw", [
    dict(n_chunks=62, kmax=128, pairs=8),               # candidates exceed shared memory
    dict(n_chunks=8, kmax=32, pairs=8, share=257),      # too many blocks for one workgroup
    dict(n_chunks=32, kmax=32, pairs=8, num_pages=PAGE_LIMIT),  # page ids do not fit the keys
    dict(n_chunks=62, kmax=0, pairs=1, resident=64),    # one pair does not fit the device
])
def test_three_launch_fallback(driver, kw):
    assert driver([case(**kw)])[0][0] == 0


def test_every_single_launch_fits_and_takes_the_fewest_rounds(driver):
    cases = []
    for resident in (256, 512, 768):
        for xcds in (0, 8):
            for n_chunks in (1, 2, 3, 8, 16, 21, 32, 33, 62):
                for pairs in (1, 2, 7, 8, 16, 64, 128):
                    cases.append(case(n_chunks, 0, pairs, resident=resident, xcds=xcds))
    results = driver(cases)
    n_single = 0
    for c, (single, n_val, bg_round, n_xcd) in zip(cases, results):
        n_chunks, resident, pairs, xcds = c[0], c[7], c[8], c[9]
        feasible = [nv for nv in range(-(-n_chunks // 4), n_chunks + 1) if resident // (n_chunks + nv) >= 1]
        assert bool(single) == bool(feasible), c
        if not single:
            continue
        n_single += 1
        W = n_chunks + n_val
        assert -(-n_chunks // 4) <= n_val <= n_chunks, c
        assert 1 <= bg_round <= pairs, c
        assert bg_round * W <= resident, c            # the whole grid is resident
        if n_xcd:
            assert n_xcd == xcds
            assert -(-bg_round // n_xcd) * W <= resident // n_xcd, c   # and each XCD's share
        best = min(-(-pairs // min(pairs, resident // (n_chunks + nv))) for nv in feasible)
        assert rounds_of(n_chunks, n_val, bg_round, pairs) == best, c
    assert n_single > 100


def test_more_rounds_than_allowed_take_three_launches(driver):
    # 128K tokens (32 chunks) per pair on 512 resident slots: 8 pairs take one
    # round, 16 two, 32 four; 16 sequences of 64K (16 chunks) and 8 KV heads
    # (128 pairs) take six
    got = driver([case(32, 32, 8, max_rounds=2), case(32, 32, 16, max_rounds=2),
                  case(32, 32, 32, max_rounds=2), case(16, 64, 128, max_rounds=2)])
    assert [g[0] for g in got] == [1, 1, 0, 0]
    assert got[1][2] == 8  # two rounds of 8 pairs
