// hf_window.h -- bookkeeping of the library-managed sliding window (host only).
//
// The window of a streaming layer keeps the latest `win` tokens, the current chunk
// included; tokens that leave it go to the linear state (Hybrid Forcing, [EN] 2.A.1
// "Linear Temporal Attention" and 2.A.2 "Block-Sparse Sliding Window Attention").
// Their K and V rows live in a caller-owned ring of `cap` rows per head. Tokens are
// numbered by their absolute index in the stream; ring row r holds token base + r.
// The ring holds the tokens [ev, hi + cur): ev is the next token the linear state
// will absorb, [ev, hi) are past chunks and [hi, hi + cur) is the current chunk.
// When the next chunk would run past the end of the ring, the tokens that leave
// the window are absorbed and the rest of the window is copied to the front
// ("slide"); with cap >= 2 * win the copy's source and destination never overlap.
//
// Plain integer arithmetic with no HIP dependence, so that host tests can build
// and exercise it on its own.
#pragma once

#include <stdint.h>

namespace hf {

struct Window {
  int64_t cap = 0;   // ring rows per head (>= 2 * win)
  int64_t win = 0;   // window tokens
  int64_t base = 0;  // token held in ring row 0
  int64_t hi = 0;    // end of the past chunks
  int64_t cur = 0;   // tokens of the current chunk (0 before the first chunk)
};

inline int64_t window_start(int64_t end, int64_t win, int64_t ev) {
  return end - win > ev ? end - win : ev;
}

// What starting a chunk of n tokens does. The current chunk joins the past
// (new_hi); the window then ends at new_hi + n and starts at ws. If the ring is
// full (slide), tokens [ev, ws) are absorbed from ring row absorb_row first and
// ring rows [copy_src_row, copy_src_row + copy_rows) move to rows [0, copy_rows);
// the token in ring row 0 becomes new_base. The chunk goes to ring row slot_row.
struct BeginPlan {
  int64_t new_hi, ws;
  bool slide;
  int64_t absorb_row, absorb_n;
  int64_t copy_src_row, copy_rows;
  int64_t new_base, slot_row;
};

// False if the chunk is empty or longer than the window, if ev is not a held
// token boundary, or if more than max_ev tokens would wait for the absorb.
inline bool plan_begin(const Window& w, int64_t ev, int64_t n, int64_t max_ev, BeginPlan* p) {
  if (n < 1 || n > w.win) return false;
  const int64_t new_hi = w.hi + w.cur;
  if (ev < w.base || ev > new_hi) return false;
  const int64_t end = new_hi + n;
  const int64_t ws = window_start(end, w.win, ev);
  if (ws - ev > max_ev) return false;
  p->new_hi = new_hi;
  p->ws = ws;
  p->slide = end - w.base > w.cap;
  p->absorb_row = ev - w.base;
  p->absorb_n = p->slide ? ws - ev : 0;
  p->copy_src_row = ws - w.base;
  p->copy_rows = p->slide ? new_hi - ws : 0;
  p->new_base = p->slide ? ws : w.base;
  p->slot_row = new_hi - p->new_base;
  return true;
}

inline void apply_begin(Window* w, const BeginPlan& p, int64_t n) {
  w->base = p.new_base;
  w->hi = p.new_hi;
  w->cur = n;
}

// The window an attend call sees: tokens [ws, ws + n_kv) from ring row win_row,
// after absorbing tokens [ev, ws) (ev_n of them) from ring row ev_row.
struct AttendView {
  int64_t ws, n_kv, win_row, ev_row, ev_n;
};

inline AttendView attend_view(const Window& w, int64_t ev) {
  AttendView v;
  const int64_t end = w.hi + w.cur;
  v.ws = window_start(end, w.win, ev);
  v.n_kv = end - v.ws;
  v.win_row = v.ws - w.base;
  v.ev_row = ev - w.base;
  v.ev_n = v.ws - ev;
  return v;
}

}  // namespace hf
