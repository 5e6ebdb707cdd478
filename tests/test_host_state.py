"""Host bookkeeping of the library (csrc/qs_state.h), on the CPU.

The header is compiled with g++ (and AddressSanitizer / UBSan) into a small driver; random
append / rollback / flush / attend scripts are replayed on it and on the CPU oracle, and the
status codes and every (layer, sequence) counter must agree after each command.  The work plan
and the arena layout are checked against their invariants.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import OracleCache, OracleError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "state_driver.cpp")
BIN = os.path.join(ROOT, "tests", "host", "state_driver")
G = 128


@pytest.fixture(scope="module")
def driver():
    oracle.build(force=False)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           SRC, "-o", BIN])
    return BIN


def run(driver, lines):
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       check=True)
    return r.stdout.splitlines()


def parse_state(line, L, B):
    parts = line.split()
    assert parts[0] == "status"
    st = int(parts[1])
    cells = [tuple(int(x) for x in c.split(",")) for c in parts[2:]]
    assert len(cells) == L * B
    return st, cells


def oracle_cells(o, L, B):
    out = []
    for l in range(L):
        nq, nt, hd = o.state(l)
        out += [(int(nq[b]), int(nt[b]), int(hd[b])) for b in range(B)]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_random_scripts_match_oracle_bookkeeping(driver, seed):
    rng = np.random.default_rng(seed)
    L, B, H, D, T, gamma = 2, 3, 1, 64, 4 * G, 5
    o = OracleCache(L, B, H, D, G, T, gamma)
    cmds = [f"create {L} {B} {H} {D} {G} {T} {gamma} 8"]
    expect = []
    for _ in range(400):
        kind = rng.choice(["append", "append", "rollback", "flush", "attend", "prefill"])
        layer = int(rng.integers(-1 if kind in ("rollback", "flush") else 0, L))
        try:
            if kind == "append":
                n_max = int(rng.choice([1, 5, 40, G, G + 1, 2 * G + 1]))
                n = [int(rng.integers(0, n_max + 1)) for _ in range(B)]
                cmds.append(f"append {layer} {n_max} " + " ".join(map(str, n)))
                z = np.zeros((B, n_max, H, D), np.float16)
                o.append(layer, z, z, n)
            elif kind == "prefill":
                if rng.random() < 0.6:                 # often empty the tails first, so that
                    d = [int(x) for x in o.state(layer)[1]]  # the prompt is accepted
                    cmds.append(f"rollback {layer} " + " ".join(map(str, d)))
                    o.rollback(layer, d)
                    expect.append((0, oracle_cells(o, L, B)))
                n_max = int(rng.choice([0, 3, G, G + 7, 3 * G + 1]))
                n = [int(rng.choice([0, int(rng.integers(0, n_max + 1))])) for _ in range(B)]
                cmds.append(f"prefill {layer} {n_max} " + " ".join(map(str, n)))
                z = np.zeros((B, n_max, H, D), np.float16)
                o.prefill(layer, z, z, n)
            elif kind == "rollback":
                d = [int(rng.integers(0, 8)) for _ in range(B)]
                cmds.append(f"rollback {layer} " + " ".join(map(str, d)))
                o.rollback(layer, d)
            elif kind == "flush":
                mt = int(rng.choice([0, G, G + 3, 2 * G, 2 * G + 1]))
                cmds.append(f"flush {layer} {mt}")
                o.flush(layer, mt)
            else:
                m = int(rng.integers(0, gamma + 3))
                draft = int(rng.integers(0, 2))
                cmds.append(f"attend {layer} {m} {draft}")
                q = np.zeros((B, H, D) if draft else (B, max(m, 1), H, D), np.float16)
                if draft:
                    o.attend_draft(layer, q)
                elif m == 0:
                    raise OracleError(1, "m = 0")
                else:
                    o.attend_verify(layer, q)
            status = 0
        except OracleError as e:
            status = e.code
        expect.append((status, oracle_cells(o, L, B)))
    out = run(driver, cmds)
    assert out[0].startswith("status 0") and len(out) == len(expect) + 1
    for i, (line, (st, cells)) in enumerate(zip(out[1:], expect)):
        got_st, got_cells = parse_state(line, L, B)
        assert got_st == st, f"command {cmds[i + 1]!r}: status {got_st} vs oracle {st}"
        assert got_cells == cells, f"command {cmds[i + 1]!r}: {got_cells} vs oracle {cells}"


def test_invalid_configs_rejected(driver):
    bad = ["create 0 1 1 64 128 128 4 8", "create 1 65 1 64 128 128 4 8",
           "create 1 1 1 96 128 128 4 8", "create 1 1 1 64 64 128 4 8",
           "create 1 1 1 64 128 200 4 8", "create 1 1 1 64 128 128 16 8",
           "create 1 1 1 64 128 128 4 3"]
    for line in bad:
        assert run(driver, [line])[0].startswith("status 1"), line


def test_plan_covers_every_group(driver):
    rng = np.random.default_rng(7)
    for _ in range(20):
        B = int(rng.integers(1, 9))
        H = int(rng.choice([1, 8, 32]))
        T = 300 * G
        lens = [int(rng.integers(0, 300 * G)) for _ in range(B)]
        cmds = [f"create 1 {B} {H} 128 {G} {T} 4 8"]
        pos = 0
        while pos < max(lens):                      # prefill by append/flush
            n = [max(0, min(G, L - pos)) for L in lens]
            cmds.append(f"append 0 {G} " + " ".join(map(str, n)))
            cmds.append("flush 0 128")
            pos += G
        target = int(rng.choice([256, 4096]))
        cmds.append(f"plan 0 {target}")
        out = run(driver, cmds)
        assert out[-1].startswith("plan")
        p = list(map(int, out[-1].split()[1:]))
        cg, items = p[0], p[1:]
        assert cg >= 1
        total = 0
        for b in range(B):
            qi, ti = items[2 * b], items[2 * b + 1]
            ng, nt = lens[b] // G, lens[b] % G
            assert qi == -(-ng // cg) and qi <= 256         # every group, whole-group chunks
            assert ti == -(-nt // 64)
            total += qi
        groups = sum(L // G for L in lens)
        if groups:
            # the smallest chunk that fits the target (and caps the splits at 256 per sequence)
            maxg = max(L // G for L in lens)
            fits = lambda c: sum(H * -(-(L // G) // c) for L in lens) <= target
            lo = max(1, -(-groups * H // target), -(-maxg // 256))
            assert cg >= lo and (fits(cg) or cg >= maxg)
            assert cg == lo or not fits(cg - 1)


@pytest.mark.parametrize("meta_fp16", [0, 1])
def test_layout_sections(driver, meta_fp16):
    out = run(driver, [f"create 2 3 4 128 128 1024 6 8 {meta_fp16}", "layout"])[-1].split()[1:]
    uk, lk, uv, lv, km, vm, tk, tv, work, state, total = map(int, out)
    offs = [uk, lk, uv, lv, km, vm, tk, tv, work, state, total]
    assert offs == sorted(offs) and all(x % 256 == 0 for x in offs)
    lbh, T, D = 2 * 3 * 4, 1024, 128
    mb = 4 if meta_fp16 else 8        # bytes of a (scale, zero-point / offset) pair
    assert lk - uk == uv - lk == lbh * T * D // 2
    assert lv - uv == km - lv == lbh * (T // G) * D * G // 2
    assert vm - km == lbh * (T // G) * D * mb
    assert tk - vm == lbh * T * mb
    assert tv - tk == work - tv == lbh * 2 * G * D * 2
    assert state - work == 3 * 4 * (256 + 4) * 7 * (D + 4) * 4
    # device-mode counters: 4 int32 per (layer, sequence) and the error word, 256-byte aligned
    assert total - state == -(-(2 * 3 * 4 + 1) * 4 // 256) * 256
