"""Host checks of the managed window's bookkeeping (hybrid_linear_block_amd/csrc/hf_window.h).

A small C++ driver built with g++ runs the header's plan over sequences of chunk
starts and attend calls; this test replays every plan on a model of the ring that
records which token each row holds, and checks what the method needs ([EN] 2.A.2:
attention over the latest window of tokens; [EN] 2.A.1: what leaves the window goes
to the linear state): each attend sees exactly the last `win` tokens (the current
chunk included) in consecutive ring rows, every token is absorbed exactly once, in
stream order, from a row that still holds it, and the slide's copy never overlaps
itself. No GPU is needed.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "hybrid_linear_block_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "hf_window.h"
int main() {
  long long cap, win, ev, max_ev;
  if (std::scanf("%lld %lld %lld %lld", &cap, &win, &ev, &max_ev) != 4) return 2;
  hf::Window w;
  w.cap = cap; w.win = win; w.base = w.hi = ev;
  char op;
  while (std::scanf(" %c", &op) == 1) {
    if (op == 'B') {
      long long n;
      if (std::scanf("%lld", &n) != 1) return 2;
      hf::BeginPlan p;
      if (!hf::plan_begin(w, ev, n, max_ev, &p)) { std::printf("reject\n"); continue; }
      std::printf("B %lld %lld %d %lld %lld %lld %lld %lld %lld\n", (long long)p.new_hi,
                  (long long)p.ws, p.slide ? 1 : 0, (long long)p.absorb_row,
                  (long long)p.absorb_n, (long long)p.copy_src_row, (long long)p.copy_rows,
                  (long long)p.new_base, (long long)p.slot_row);
      ev += p.absorb_n;
      hf::apply_begin(&w, p, n);
    } else {
      hf::AttendView v = hf::attend_view(w, ev);
      std::printf("A %lld %lld %lld %lld %lld\n", (long long)v.ws, (long long)v.n_kv,
                  (long long)v.win_row, (long long)v.ev_row, (long long)v.ev_n);
      ev += v.ev_n;
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("window_plan")
    src = d / "drv.cc"
    src.write_text(DRIVER)
    exe = d / "drv"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", HEADER_DIR, str(src), "-o", str(exe)],
                   check=True)
    return str(exe)


def run(driver, cap, win, ev0, max_ev, ops):
    text = f"{cap} {win} {ev0} {max_ev}\n" + "\n".join(ops) + "\n"
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True)
    return out.stdout.split("\n")[:-1]


def replay(lines, ops, cap, win, ev0, max_ev):
    """Model of the ring (token held by each row, -1 = nothing yet) driven by the
    plans; asserts the invariants (a rejected chunk start must be empty, longer than
    the window or leave more than max_ev tokens waiting for the absorb) and returns
    (absorbed tokens, slides, next token to absorb, start of the current chunk)."""
    ring = np.full(cap, -1, dtype=np.int64)
    ev, nxt, absorbed, slides = ev0, ev0, [], 0
    chunk_end = ev0  # one past the last token of the current chunk
    for op, line in zip(ops, lines):
        f = line.split()
        if op.startswith("B"):
            n = int(op.split()[1])
            if f[0] == "reject":
                assert n < 1 or n > win or max(ev, chunk_end + n - win) - ev > max_ev
                continue
            assert f[0] == "B", line
            assert 1 <= n <= win and max(ev, chunk_end + n - win) - ev <= max_ev
            new_hi, ws, slide, arow, an, src, rows, new_base, slot = map(int, f[1:])
            assert new_hi == chunk_end
            end = chunk_end + n
            assert ws == max(ev, end - win)
            if slide:
                slides += 1
                assert np.array_equal(ring[arow:arow + an], np.arange(ev, ev + an))
                absorbed.extend(range(ev, ev + an))
                ev += an
                assert ev == ws
                assert src >= rows  # disjoint copy
                assert np.array_equal(ring[src:src + rows], np.arange(ws, ws + rows))
                ring[0:rows] = ring[src:src + rows].copy()
                assert new_base == ws
            else:
                assert an == 0 and rows == 0
            assert 0 <= slot and slot + n <= cap
            assert slot == new_hi - new_base
            ring[slot:slot + n] = np.arange(chunk_end, end)  # the caller writes the chunk
            nxt, chunk_end = chunk_end, end
        else:
            assert f[0] == "A", line
            ws, n_kv, wrow, erow, en = map(int, f[1:])
            assert ws == max(ev, chunk_end - win) and ws + n_kv == chunk_end
            assert n_kv == min(win, chunk_end - ev)
            assert np.array_equal(ring[wrow:wrow + n_kv], np.arange(ws, chunk_end))
            assert np.array_equal(ring[erow:erow + en], np.arange(ev, ev + en))
            absorbed.extend(range(ev, ev + en))
            ev += en
    return absorbed, slides, ev, nxt


@pytest.mark.parametrize("chunk,win,ring_mult", [(3, 9, 2), (4680, 14040, 2), (4680, 14040, 3),
                                                  (64, 128, 2), (5, 5, 2), (7, 20, 5)])
def test_streaming_chunks(driver, chunk, win, ring_mult):
    """Equal chunks, one or two attends per chunk: the window and the absorbed
    tokens follow the stream order of the method, and the ring slides."""
    cap = ring_mult * win
    ops = []
    for t in range(40):
        ops.append(f"B {chunk}")
        ops += ["A"] * (1 + t % 2)
    lines = run(driver, cap, win, 0, chunk, ops)
    assert "reject" not in lines
    absorbed, slides, ev, _ = replay(lines, ops, cap, win, 0, chunk)
    end = 40 * chunk
    assert absorbed == list(range(0, ev)) and ev == max(0, end - win)
    assert slides >= 1


def test_random_chunk_sizes_and_start(driver):
    rng = np.random.default_rng(5)
    rejected = accepted = 0
    for trial in range(30):
        win = int(rng.integers(1, 200))
        cap = int(rng.integers(2 * win, 5 * win + 1))
        ev0 = int(rng.integers(0, 10**12))
        ops = []
        for _ in range(60):
            ops.append(f"B {int(rng.integers(1, win + 1))}")
            ops += ["A"] * int(rng.integers(0, 3))
        max_ev = int(rng.integers(1, 2 * win + 1))
        lines = run(driver, cap, win, ev0, max_ev, ops)
        absorbed, _, ev, _ = replay(lines, ops, cap, win, ev0, max_ev)
        assert absorbed == list(range(ev0, ev))
        rejected += lines.count("reject")
        accepted += sum(1 for x in lines if x.startswith("B"))
    assert rejected > 0 and accepted > 2 * rejected, (accepted, rejected)


def test_rejections(driver):
    # empty chunk, chunk longer than the window, and too many tokens waiting for the
    # absorb (two chunk starts without an attend between them)
    lines = run(driver, 20, 10, 0, 4, ["B 0", "B 11", "B 10", "B 4", "B 4", "B 4"])
    assert lines[0] == "reject" and lines[1] == "reject"
    assert lines[2].startswith("B") and lines[3].startswith("B")
    # 10 + 4 tokens with a window of 10: 4 wait; 4 more would make 8 > max_ev = 4
    assert lines[4] == "reject"
