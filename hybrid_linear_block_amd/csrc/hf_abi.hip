// hf_abi.hip -- the extern "C" entry points of libhf (declared in include/hf.h).
//
// Host side only: argument validation (always before any HIP call, so that an
// invalid call enqueues nothing), the workspace layout, the eviction-sequence
// check and the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/hf.h"
#include "hf_launch.h"
#include "hf_window.h"

struct hf_state {
  hf_config cfg;
  float* S;
  float* z;
  char* ws;
  size_t ws_bytes;
  int64_t next_ev;
  int device;
  float scale;
  int nqb_cap, nkb_cap;
  float* pooled_q;
  float* pooled_k;
  int32_t* sel;
  float* partials;
  // Tokens whose partial states an ahead call left in `partials` for the next call to
  // reduce into S and z (0: none pending).
  int64_t pend_n = 0;
  // Managed window: partial states formed ahead, in an attention launch, for the tokens
  // [spec_lo, spec_lo + spec_n) that leave the window at the next chunk if it has the
  // current chunk's size. They are not absorbed yet: the next absorb of exactly those
  // tokens reduces them, anything else that writes `partials` drops them.
  int64_t spec_lo = 0, spec_n = 0;
  uint16_t* s_split;  // bf16 hi/lo split of S (bf16 states), kept in step with S
  // Cache of 8-token key sums for the cached calls: ring of kc_cap groups per head;
  // the absolute groups [kc_lo, kc_hi) hold the sums of the last cached window.
  float* kcache;
  int64_t kc_cap = 1, kc_lo = 0, kc_hi = 0;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;  // hf_absorb_and_attend's fork / join
  // Library-managed window over the caller's K/V ring (hf_window_attach); win_ok turns
  // false if a slide could not be enqueued whole.
  hf::Window win;
  char* k_ring = nullptr;
  char* v_ring = nullptr;
  bool win_on = false, win_ok = false;
  // Relative temporal rotation of the softmax path (hf_set_rope); rope.cs == nullptr: off.
  hf_rope rope_cfg = {};
  hf::Rope rope;
  // Per-kernel timing (hf_profile_start / hf_profile_stop).
  bool prof_on = false;
  int prof_cap = 0;
  std::vector<hipEvent_t> prof_ev[HF_KERNEL_COUNT];  // start/end pairs
  int prof_n[HF_KERNEL_COUNT] = {};
};

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == HF_BF16 ? 2 : 4; }

// Configuration check: HF_ERR_INVALID_ARG for values that are meaningless,
// HF_ERR_UNSUPPORTED for meaningful values outside the instantiated kernels.
hf_status check_config(const hf_config* c) {
  if (!c) return HF_ERR_INVALID_ARG;
  if (c->num_heads < 1 || c->head_dim < 1 || c->block_size < 1) return HF_ERR_INVALID_ARG;
  if (c->dtype != HF_BF16 && c->dtype != HF_F32) return HF_ERR_UNSUPPORTED;
  // eps > 0: an empty state (z = 0) must read as an exactly zero linear term, and
  // 0 / (0 + eps) is 0 only for eps > 0.
  if (!(c->eps > 0.f) || !std::isfinite(c->eps)) return HF_ERR_INVALID_ARG;
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale)) return HF_ERR_INVALID_ARG;
  if (c->max_n_q < 1 || c->max_n_kv < 1 || c->max_n_ev < 0 || c->max_top_k < 1)
    return HF_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return HF_ERR_UNSUPPORTED;
  if (c->dtype == HF_BF16 && c->block_size != 64) return HF_ERR_UNSUPPORTED;
  if (c->dtype == HF_F32 && c->block_size != 16 && c->block_size != 64) return HF_ERR_UNSUPPORTED;
  if (ceil_div(c->max_n_kv, c->block_size) > hf::kMaxKeyBlocks) return HF_ERR_UNSUPPORTED;
  if (ceil_div(c->max_n_q, c->block_size) > (int64_t)1 << 24) return HF_ERR_UNSUPPORTED;
  // Launch sizes are 32-bit products of the head count and the block counts (a
  // workgroup or wave per (head, block), up to a few per block in the backward), so
  // their sum per head times the heads stays below 2^26.
  if ((int64_t)c->num_heads *
          (ceil_div(c->max_n_q, c->block_size) + ceil_div(c->max_n_kv, c->block_size)) >
      (int64_t)1 << 26)
    return HF_ERR_UNSUPPORTED;
  if (c->max_top_k > ceil_div(c->max_n_kv, c->block_size)) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

struct Layout {
  size_t pooled_q, pooled_k, sel, partials, s_split, kcache, total;
  int64_t kc_cap;  // groups per head of the key-sum cache (a power of two)
};

Layout layout(const hf_config* c) {
  const size_t H = (size_t)c->num_heads, d = (size_t)c->head_dim;
  const size_t nqb = (size_t)ceil_div(c->max_n_q, c->block_size);
  const size_t nkb = (size_t)ceil_div(c->max_n_kv, c->block_size);
  Layout L;
  size_t off = 0;
  L.pooled_q = off;
  off += round_up(H * nqb * d * 4);
  L.pooled_k = off;
  off += round_up(H * nkb * d * 4);
  L.sel = off;
  off += round_up(H * nqb * (size_t)c->max_top_k * 4);
  L.partials = off;
  off += round_up(hf::absorb_partial_floats((int)H, (int)d) * 4);
  L.s_split = off;
  if (c->dtype == HF_BF16) off += round_up(H * 2 * d * d * 2);
  // The cache holds every 8-token group of the largest window.
  L.kc_cap = 1;
  while (L.kc_cap < ceil_div(c->max_n_kv, 8)) L.kc_cap *= 2;
  L.kcache = off;
  off += round_up(H * (size_t)L.kc_cap * d * 4);
  L.total = off;
  return L;
}

// Runs `fn` with the state's device current, restoring the caller's device.
template <typename F>
hf_status on_device(int device, F fn) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return HF_ERR_HIP;
  if (cur != device && hipSetDevice(device) != hipSuccess) return HF_ERR_HIP;
  const hipError_t e = fn();
  if (cur != device) (void)hipSetDevice(cur);
  return e == hipSuccess ? HF_OK : HF_ERR_HIP;
}

void prof_release(hf_state* st) {
  for (int k = 0; k < HF_KERNEL_COUNT; ++k) {
    for (hipEvent_t e : st->prof_ev[k]) (void)hipEventDestroy(e);
    st->prof_ev[k].clear();
    st->prof_n[k] = 0;
  }
  st->prof_on = false;
  st->prof_cap = 0;
}

void release_events(hf_state* st) {
  if (st->ev_fork) (void)hipEventDestroy(st->ev_fork);
  if (st->ev_join) (void)hipEventDestroy(st->ev_join);
  st->ev_fork = st->ev_join = nullptr;
}

// Launch `fn` (one kernel) on stream s, bracketed by profiling events if enabled.
template <typename F>
hipError_t timed(hf_state* st, int kernel, hipStream_t s, F fn) {
  const bool rec = st->prof_on && st->prof_n[kernel] < st->prof_cap;
  const int i = st->prof_n[kernel];
  if (rec) {
    const hipError_t e = hipEventRecord(st->prof_ev[kernel][2 * i], s);
    if (e != hipSuccess) return e;
  }
  const hipError_t r = fn();
  if (rec && r == hipSuccess) {
    const hipError_t e = hipEventRecord(st->prof_ev[kernel][2 * i + 1], s);
    if (e != hipSuccess) return e;
    st->prof_n[kernel] = i + 1;
  }
  return r;
}

hf_status check_tensor(const void* p, int64_t n, int64_t head_stride, const hf_config& c) {
  if (!p || !aligned16(p)) return HF_ERR_INVALID_ARG;
  if (head_stride < n * c.head_dim) return HF_ERR_INVALID_ARG;
  if ((head_stride * (int64_t)elem_size(c.dtype)) % 16 != 0) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

// ---- Relative temporal rotation -------------------------------------------------------
struct RopeLayout {
  size_t table, k_copy, total;
  int npos;
};

RopeLayout rope_layout(const hf_config& c, const hf_rope& r) {
  const int64_t frames = ceil_div(c.max_n_kv, r.tokens_per_frame);
  RopeLayout L;
  L.npos = (int)((frames - 1 < r.cap ? frames - 1 : r.cap) + 1);
  L.table = 0;
  L.k_copy = round_up((size_t)L.npos * (size_t)(r.rot_dims / 2) * 8);
  L.total = L.k_copy + round_up((size_t)c.num_heads * (size_t)c.max_n_kv * (size_t)c.head_dim *
                                elem_size(c.dtype));
  return L;
}

hf_status check_rope(const hf_config& c, const hf_rope* r) {
  if (!r) return HF_ERR_INVALID_ARG;
  if (r->rot_dims < 0 || r->rot_dims % 2 != 0 || r->rot_dims > c.head_dim) return HF_ERR_INVALID_ARG;
  if (!(r->theta_base > 0.f) || !std::isfinite(r->theta_base)) return HF_ERR_INVALID_ARG;
  if (r->tokens_per_frame < 8 || r->tokens_per_frame > INT32_MAX || r->cap < 0)
    return HF_ERR_INVALID_ARG;
  return HF_OK;
}

// ---- Scratch of hf_attend_chunk_noalloc ---------------------------------------------
// A file-scope device array: every device the library runs on holds its own copy
// until the process ends. Host code never passes `hf_noalloc_scratch` itself to a
// kernel (on the host that name is only a stand-in, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) unsigned char hf_noalloc_scratch[HF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (the device is current); nullptr on error.
char* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(hf_noalloc_scratch)) != hipSuccess || !p)
      return nullptr;
    g_scratch_ptr[device] = static_cast<char*>(p);
  }
  return g_scratch_ptr[device];
}

// Scratch layout of one call: pooled query and key means, the selection (if the
// caller passes none) and, for bf16, the hi/lo split of S.
struct NoallocLayout {
  size_t pooled_q, pooled_k, sel, s_split, total;
};

NoallocLayout noalloc_layout(const hf_config& c, int64_t n_q, int64_t n_kv, int32_t top_k) {
  const size_t H = (size_t)c.num_heads, d = (size_t)c.head_dim;
  const size_t nqb = (size_t)ceil_div(n_q, c.block_size), nkb = (size_t)ceil_div(n_kv, c.block_size);
  NoallocLayout L;
  size_t off = 0;
  L.pooled_q = off;
  off += round_up(H * nqb * d * 4);
  L.pooled_k = off;
  off += round_up(H * nkb * d * 4);
  L.sel = off;
  off += round_up(H * nqb * (size_t)top_k * 4);
  L.s_split = off;
  if (c.dtype == HF_BF16) off += round_up(H * 2 * d * d * 2);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t hf_workspace_bytes(const hf_config* cfg) {
  if (check_config(cfg) != HF_OK) return 0;
  return layout(cfg).total;
}

hf_status hf_state_init(const hf_config* cfg, float* S, float* z, void* workspace,
                        size_t ws_bytes, int zero_fill, int64_t next_ev_index, void* stream,
                        hf_state** out) {
  if (!out) return HF_ERR_INVALID_ARG;
  *out = nullptr;
  const hf_status cs = check_config(cfg);
  if (cs != HF_OK) return cs;
  if (!S || !z || !workspace || !aligned16(S) || !aligned16(z) || !aligned16(workspace))
    return HF_ERR_INVALID_ARG;
  if (next_ev_index < 0) return HF_ERR_INVALID_ARG;
  const Layout L = layout(cfg);
  if (ws_bytes < L.total) return HF_ERR_INVALID_ARG;

  hf_state* st = new (std::nothrow) hf_state();
  if (!st) return HF_ERR_HIP;
  st->cfg = *cfg;
  st->S = S;
  st->z = z;
  st->ws = static_cast<char*>(workspace);
  st->ws_bytes = ws_bytes;
  st->next_ev = next_ev_index;
  st->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                       : 1.0f / std::sqrt((float)cfg->head_dim);
  st->nqb_cap = (int)ceil_div(cfg->max_n_q, cfg->block_size);
  st->nkb_cap = (int)ceil_div(cfg->max_n_kv, cfg->block_size);
  st->pooled_q = reinterpret_cast<float*>(st->ws + L.pooled_q);
  st->pooled_k = reinterpret_cast<float*>(st->ws + L.pooled_k);
  st->sel = reinterpret_cast<int32_t*>(st->ws + L.sel);
  st->partials = reinterpret_cast<float*>(st->ws + L.partials);
  st->s_split = cfg->dtype == HF_BF16 ? reinterpret_cast<uint16_t*>(st->ws + L.s_split) : nullptr;
  st->kcache = reinterpret_cast<float*>(st->ws + L.kcache);
  st->kc_cap = L.kc_cap;
  if (hipGetDevice(&st->device) != hipSuccess) {
    delete st;
    return HF_ERR_HIP;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t H = (size_t)cfg->num_heads, d = (size_t)cfg->head_dim;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    hipError_t e = hipSuccess;
    if (zero_fill) e = hf::launch_fill_zero(S, H * d * d * 4, s);
    if (e == hipSuccess && zero_fill) e = hf::launch_fill_zero(z, H * d * 4, s);
    if (e == hipSuccess && st->s_split)
      e = zero_fill ? hf::launch_fill_zero(st->s_split, H * 2 * d * d * 2, s)
                    : hf::launch_split_state((int)H, (int)d, S, st->s_split, s);
    return e;
  });
  const hf_status re = r != HF_OK ? r : on_device(st->device, [&]() -> hipError_t {
    hipError_t e = hipEventCreateWithFlags(&st->ev_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->ev_join, hipEventDisableTiming);
    return e;
  });
  if (re != HF_OK) {
    release_events(st);
    delete st;
    return re;
  }
  *out = st;
  return HF_OK;
}

static hf_status check_absorb(const hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                              int64_t ev_head_stride, int64_t ev_index) {
  const hf_config& c = st->cfg;
  if (n_ev < 0 || n_ev > c.max_n_ev) return HF_ERR_INVALID_ARG;
  if (n_ev > 0) {
    hf_status e = check_tensor(k_ev, n_ev, ev_head_stride, c);
    if (e == HF_OK) e = check_tensor(v_ev, n_ev, ev_head_stride, c);
    if (e != HF_OK) return e;
  }
  return ev_index != st->next_ev ? HF_ERR_STATE : HF_OK;
}

// The reduce of the partial states that hf_absorb_and_attend_ahead left in the
// workspace, if any, on stream s. Every call that reads or writes S, z or the
// workspace's partial states completes a pending absorb first.
static hipError_t flush_pending(hf_state* st, hipStream_t s) {
  if (st->pend_n == 0) return hipSuccess;
  const hf_config& c = st->cfg;
  const hipError_t e = timed(st, HF_KERNEL_ABSORB, s, [&]() {
    return hf::launch_absorb_reduce(c.dtype, c.num_heads, c.head_dim, st->pend_n, st->partials,
                                    st->S, st->z, st->s_split, s);
  });
  if (e == hipSuccess) st->pend_n = 0;
  return e;
}

// The absorb kernels on stream s (n_ev > 0); the caller has validated everything.
static hipError_t enqueue_absorb(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                                 int64_t ev_head_stride, hipStream_t s) {
  const hf_config& c = st->cfg;
  const hipError_t e = flush_pending(st, s);
  if (e != hipSuccess) return e;
  st->spec_n = 0;  // its partial states take the buffer
  return timed(st, HF_KERNEL_ABSORB, s, [&]() {
    return hf::launch_absorb(c.dtype, c.num_heads, c.head_dim, k_ev, v_ev, n_ev, ev_head_stride,
                             st->S, st->z, st->partials, st->s_split, s);
  });
}

hf_status hf_absorb_evicted(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                            int64_t ev_head_stride, int64_t ev_index, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  const hf_status e = check_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, ev_index);
  if (e != HF_OK || n_ev == 0) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hf_status r =
      on_device(st->device, [&]() { return enqueue_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, s); });
  if (r == HF_OK) st->next_ev += n_ev;
  return r;
}

static hf_status check_attend(const hf_state* st, const void* q, int64_t n_q, int64_t q_hs,
                              const void* k_win, int64_t n_kv, int64_t kv_hs) {
  const hf_config& c = st->cfg;
  if (n_q < 0 || n_kv < 1) return HF_ERR_INVALID_ARG;
  if (n_q > c.max_n_q || n_kv > c.max_n_kv) return HF_ERR_INVALID_ARG;
  hf_status e = n_q > 0 ? check_tensor(q, n_q, q_hs, c) : HF_OK;
  if (e == HF_OK) e = check_tensor(k_win, n_kv, kv_hs, c);
  return e;
}

static hf_status check_attend_all(const hf_state* st, const void* q, int64_t n_q, int64_t q_hs,
                                  const void* k_win, const void* v_win, int64_t n_kv,
                                  int64_t kv_hs, int32_t top_k, const void* out, int64_t out_hs,
                                  const int32_t* sel_out) {
  const hf_config& c = st->cfg;
  hf_status e = check_attend(st, q, n_q, q_hs, k_win, n_kv, kv_hs);
  if (e == HF_OK) e = check_tensor(v_win, n_kv, kv_hs, c);
  if (e == HF_OK && n_q > 0) e = check_tensor(out, n_q, out_hs, c);
  if (e != HF_OK) return e;
  const int64_t nkb = ceil_div(n_kv, c.block_size);
  if (top_k < 1 || top_k > nkb || top_k > c.max_top_k) return HF_ERR_INVALID_ARG;
  if (sel_out && (reinterpret_cast<uintptr_t>(sel_out) & 3u)) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

// Shapes an attend call needs when the rotation is on: the window holds whole frames
// and the chunk's queries are its last rows.
static hf_status check_rope_shapes(const hf_state* st, int64_t n_q, int64_t n_kv) {
  if (!st->rope.cs) return HF_OK;
  if (n_kv % st->rope.tpf != 0 || n_q > n_kv) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

// Window of a cached call: it starts on an 8-token group of the stream and holds
// whole groups (the block size is a multiple of 8 in every configuration).
static hf_status check_window(int64_t win_index, int64_t n_kv) {
  if (win_index < 0 || win_index % 8 != 0 || n_kv % 8 != 0) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

// The key-sum cache for a call over the window [win_index, win_index + n_kv).
static hf::KeyCache key_cache(const hf_state* st, int64_t win_index) {
  hf::KeyCache kc;
  kc.ring = st->kcache;
  kc.cap = st->kc_cap;
  kc.g0 = win_index / 8;
  kc.lo = st->kc_lo;
  kc.hi = st->kc_hi;
  return kc;
}

// Evicted tokens that an attend call absorbs in its own launches.
struct FusedAbsorb {
  const void* k_ev;
  const void* v_ev;
  int64_t n_ev;  // > 0
  int64_t head_stride;
};

// Block pooling, selection and attention on stream s (n_q > 0), validated by the
// caller; with `join`, the attention waits for that event. With `fa`, the absorb of
// its tokens runs inside the first two launches: the partial states next to the
// pooling, the reduce next to the selection, so S and z hold the new tokens before
// the attention reads them; *absorbed tells whether the reduce was enqueued. A pending
// absorb (an ahead call's) is reduced in the selection launch (before the pooling
// launch if `fa` needs the partial-state buffer). With `next`, the partial states of
// those tokens are formed in the attention launch (bf16; fp32: a launch after it) and
// left pending; *formed tells whether they were enqueued.
static hipError_t enqueue_attend(hf_state* st, const void* q, int64_t n_q, int64_t q_hs,
                                 const void* k_win, const void* v_win, int64_t n_kv,
                                 int64_t kv_hs, int32_t top_k, void* out, int64_t out_hs,
                                 int32_t* sel_out, hipStream_t s, hipEvent_t join,
                                 const FusedAbsorb* fa = nullptr, bool* absorbed = nullptr,
                                 const hf::KeyCache* kc = nullptr,
                                 const FusedAbsorb* next = nullptr, bool* formed = nullptr) {
  const hf_config& c = st->cfg;
  if (absorbed) *absorbed = false;
  if (formed) *formed = false;
  if (fa && st->pend_n > 0) {
    const hipError_t e = flush_pending(st, s);
    if (e != hipSuccess) return e;
  }
  if (fa || next) st->spec_n = 0;  // partial states of this call take the buffer
  const int64_t reduce_n = fa ? 0 : st->pend_n;
  const int nqb = (int)ceil_div(n_q, c.block_size);
  const int nkb = (int)ceil_div(n_kv, c.block_size);
  int32_t* sel = sel_out ? sel_out : st->sel;
  // With the rotation on, the pooling rotates Q and K and writes the rotated window
  // keys, which the attention kernel reads instead of k_win (the chunk's queries are
  // the window's last n_q rows).
  hf::Rope rope = st->rope;
  if (rope.cs) rope.q_row0 = n_kv - n_q;
  hipError_t r = timed(st, HF_KERNEL_BLOCK_POOL, s, [&]() {
    const hf::KeyCache none;
    const hf::KeyCache& kcr = kc ? *kc : none;
    if (fa)
      return hf::launch_absorb_and_pool(c.dtype, c.num_heads, c.head_dim, c.block_size, fa->k_ev,
                                        fa->v_ev, fa->n_ev, fa->head_stride, st->partials, q, n_q,
                                        q_hs, k_win, n_kv, kv_hs, st->pooled_q, st->pooled_k,
                                        st->nqb_cap, st->nkb_cap, s, kcr, rope);
    return hf::launch_block_pool(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q, q_hs,
                                 k_win, n_kv, kv_hs, st->pooled_q, st->pooled_k, st->nqb_cap,
                                 st->nkb_cap, s, kcr, rope);
  });
  if (r == hipSuccess && kc) {  // the pooling launch sums (or reads) every group of the window
    st->kc_lo = kc->g0;
    st->kc_hi = kc->g0 + n_kv / 8;
  }
  if (r == hipSuccess)
    r = timed(st, HF_KERNEL_SCORE_SELECT, s, [&]() {
      const int64_t red = fa ? fa->n_ev : reduce_n;
      if (red > 0)
        return hf::launch_select_and_reduce(c.dtype, c.num_heads, c.head_dim, nqb, nkb,
                                            st->nqb_cap, st->nkb_cap, st->pooled_q, st->pooled_k,
                                            st->scale, top_k, sel, st->partials, red, st->S,
                                            st->z, st->s_split, s);
      return hf::launch_score_select(c.num_heads, c.head_dim, nqb, nkb, st->nqb_cap, st->nkb_cap,
                                     st->pooled_q, st->pooled_k, st->scale, top_k, sel, nullptr,
                                     s);
    });
  if (absorbed) *absorbed = fa && r == hipSuccess;
  if (r == hipSuccess && reduce_n > 0) st->pend_n = 0;
  if (r == hipSuccess && join) r = hipStreamWaitEvent(s, join, 0);
  // bf16: the next absorb's partial states are formed by workgroups appended to the
  // attention launch, in the slots its own workgroups leave free.
  hf::AbsorbAhead ab;
  const bool in_launch = next && c.dtype == HF_BF16;
  if (in_launch) {
    const hf::AbsorbPlan p = hf::absorb_plan(c.dtype, c.num_heads, c.head_dim, next->n_ev);
    ab.k = next->k_ev;
    ab.v = next->v_ev;
    ab.n_ev = next->n_ev;
    ab.hs = next->head_stride;
    ab.tps = p.tokens_per_split;
    ab.n_split = p.n_split;
    ab.partials = st->partials;
  }
  if (r == hipSuccess)
    r = timed(st, HF_KERNEL_SPARSE_SWA, s, [&]() {
      return hf::launch_sparse_swa(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q, q_hs,
                                   k_win, v_win, n_kv, kv_hs, sel, top_k, st->S, st->s_split,
                                   st->z, c.eps, st->scale, out, out_hs, s, rope, hf::Ragged(),
                                   ab);
    });
  if (r == hipSuccess && next && !in_launch)
    r = timed(st, HF_KERNEL_ABSORB, s, [&]() {
      return hf::launch_absorb_parts(c.dtype, c.num_heads, c.head_dim, next->k_ev, next->v_ev,
                                     next->n_ev, next->head_stride, st->partials, s);
    });
  if (formed) *formed = next && r == hipSuccess;
  return r;
}

hf_status hf_attend_chunk(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                          const void* k_win, const void* v_win, int64_t n_kv,
                          int64_t kv_head_stride, int32_t top_k, void* out,
                          int64_t out_head_stride, int32_t* sel_out, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  hf_status e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv,
                                 kv_head_stride, top_k, out, out_head_stride, sel_out);
  if (e == HF_OK) e = check_rope_shapes(st, n_q, n_kv);
  if (e != HF_OK || n_q == 0) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() {
    return enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                          out, out_head_stride, sel_out, s, nullptr);
  });
}

hf_status hf_absorb_and_attend(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                               int64_t ev_head_stride, int64_t ev_index, const void* q,
                               int64_t n_q, int64_t q_head_stride, const void* k_win,
                               const void* v_win, int64_t n_kv, int64_t kv_head_stride,
                               int32_t top_k, void* out, int64_t out_head_stride,
                               int32_t* sel_out, void* stream, void* side_stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  hf_status e = check_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, ev_index);
  if (e == HF_OK)
    e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                         out, out_head_stride, sel_out);
  if (e == HF_OK && n_q > 0) e = check_rope_shapes(st, n_q, n_kv);
  if (e != HF_OK) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t side = static_cast<hipStream_t>(side_stream);
  const bool fork = n_ev > 0 && n_q > 0 && side != nullptr && side != s;
  bool absorbed = false;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    hipError_t err = hipSuccess;
    if (fork) {
      err = hipEventRecord(st->ev_fork, s);
      if (err == hipSuccess) err = hipStreamWaitEvent(side, st->ev_fork, 0);
      if (err == hipSuccess) err = enqueue_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, side);
      absorbed = err == hipSuccess;
      if (err == hipSuccess) err = hipEventRecord(st->ev_join, side);
      if (err == hipSuccess)
        err = enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride,
                             top_k, out, out_head_stride, sel_out, s, st->ev_join);
      return err;
    }
    // One stream: the absorb runs inside the attend call's pooling and selection
    // launches; it counts as enqueued once its reduce is.
    if (n_q == 0) {
      if (n_ev > 0) {
        err = enqueue_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, s);
        absorbed = err == hipSuccess;
      }
      return err;
    }
    const FusedAbsorb fa{k_ev, v_ev, n_ev, ev_head_stride};
    return enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                          out, out_head_stride, sel_out, s, nullptr, n_ev > 0 ? &fa : nullptr,
                          &absorbed);
  });
  if (absorbed) st->next_ev += n_ev;  // the absorb is enqueued and will run
  return r;
}

hf_status hf_attend_chunk_cached(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                                 const void* k_win, const void* v_win, int64_t n_kv,
                                 int64_t kv_head_stride, int64_t win_index, int32_t top_k,
                                 void* out, int64_t out_head_stride, int32_t* sel_out,
                                 void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (st->rope.cs) return HF_ERR_UNSUPPORTED;  // rotated keys are not cached
  hf_status e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride,
                                 top_k, out, out_head_stride, sel_out);
  if (e == HF_OK && n_q > 0) e = check_window(win_index, n_kv);
  if (e != HF_OK || n_q == 0) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hf::KeyCache kc = key_cache(st, win_index);
  return on_device(st->device, [&]() {
    return enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                          out, out_head_stride, sel_out, s, nullptr, nullptr, nullptr, &kc);
  });
}

hf_status hf_absorb_and_attend_cached(hf_state* st, const void* k_ev, const void* v_ev,
                                      int64_t n_ev, int64_t ev_head_stride, int64_t ev_index,
                                      const void* q, int64_t n_q, int64_t q_head_stride,
                                      const void* k_win, const void* v_win, int64_t n_kv,
                                      int64_t kv_head_stride, int64_t win_index, int32_t top_k,
                                      void* out, int64_t out_head_stride, int32_t* sel_out,
                                      void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (st->rope.cs) return HF_ERR_UNSUPPORTED;  // rotated keys are not cached
  hf_status e = check_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, ev_index);
  if (e == HF_OK)
    e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                         out, out_head_stride, sel_out);
  if (e == HF_OK && n_q > 0) e = check_window(win_index, n_kv);
  if (e != HF_OK) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hf::KeyCache kc = key_cache(st, win_index);
  bool absorbed = false;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    if (n_q == 0) {
      hipError_t err = hipSuccess;
      if (n_ev > 0) {
        err = enqueue_absorb(st, k_ev, v_ev, n_ev, ev_head_stride, s);
        absorbed = err == hipSuccess;
      }
      return err;
    }
    const FusedAbsorb fa{k_ev, v_ev, n_ev, ev_head_stride};
    return enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                          out, out_head_stride, sel_out, s, nullptr, n_ev > 0 ? &fa : nullptr,
                          &absorbed, &kc);
  });
  if (absorbed) st->next_ev += n_ev;  // the absorb is enqueued and will run
  return r;
}

hf_status hf_absorb_and_attend_ahead(hf_state* st, const void* q, int64_t n_q,
                                     int64_t q_head_stride, const void* k_win, const void* v_win,
                                     int64_t n_kv, int64_t kv_head_stride, int64_t win_index,
                                     int32_t top_k, void* out, int64_t out_head_stride,
                                     int32_t* sel_out, const void* k_next, const void* v_next,
                                     int64_t n_next, int64_t next_head_stride,
                                     int64_t next_index, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  const hf_config& c = st->cfg;
  hf_status e = check_absorb(st, k_next, v_next, n_next, next_head_stride, next_index);
  if (e == HF_OK)
    e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                         out, out_head_stride, sel_out);
  if (e == HF_OK && n_q > 0) e = check_rope_shapes(st, n_q, n_kv);
  if (e == HF_OK && n_q > 0 && win_index >= 0)
    e = st->rope.cs ? HF_ERR_UNSUPPORTED : check_window(win_index, n_kv);  // rotated keys are not cached
  if (e != HF_OK) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hf::KeyCache kc = key_cache(st, win_index >= 0 ? win_index : 0);
  bool formed = false;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    const FusedAbsorb nx{k_next, v_next, n_next, next_head_stride};
    if (n_q == 0) {  // no attention launch to carry the partial states: a launch of their own
      hipError_t err = flush_pending(st, s);
      if (err == hipSuccess && n_next > 0) {
        st->spec_n = 0;
        err = timed(st, HF_KERNEL_ABSORB, s, [&]() {
          return hf::launch_absorb_parts(c.dtype, c.num_heads, c.head_dim, k_next, v_next, n_next,
                                         next_head_stride, st->partials, s);
        });
        formed = err == hipSuccess;
      }
      return err;
    }
    return enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                          out, out_head_stride, sel_out, s, nullptr, nullptr, nullptr,
                          win_index >= 0 ? &kc : nullptr, n_next > 0 ? &nx : nullptr, &formed);
  });
  if (formed) {  // the partial states are enqueued: the tokens count as absorbed
    st->pend_n = n_next;
    st->next_ev += n_next;
  }
  return r;
}

hf_status hf_absorb_flush(hf_state* st, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (st->pend_n == 0) return HF_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() { return flush_pending(st, s); });
}

int64_t hf_pending_ev(const hf_state* st) { return st ? st->pend_n : -1; }

hf_status hf_window_attach(hf_state* st, void* k_ring, void* v_ring, int64_t ring_tokens,
                           int64_t window_tokens) {
  if (!st || !k_ring || !v_ring || !aligned16(k_ring) || !aligned16(v_ring))
    return HF_ERR_INVALID_ARG;
  const hf_config& c = st->cfg;
  if (window_tokens < 1 || window_tokens > c.max_n_kv) return HF_ERR_INVALID_ARG;
  if (ring_tokens < 2 * window_tokens) return HF_ERR_INVALID_ARG;
  if (c.num_heads > 65535) return HF_ERR_UNSUPPORTED;  // the slide's copy grid
  st->win = hf::Window();
  st->win.cap = ring_tokens;
  st->win.win = window_tokens;
  st->win.base = st->win.hi = st->next_ev;
  st->k_ring = static_cast<char*>(k_ring);
  st->v_ring = static_cast<char*>(v_ring);
  st->win_on = st->win_ok = true;
  st->kc_lo = st->kc_hi = 0;  // cached key sums may come from other buffers
  st->spec_n = 0;
  return HF_OK;
}

hf_status hf_window_begin_chunk(hf_state* st, int64_t n, void* stream, void** k_slot,
                                void** v_slot, int64_t* head_stride) {
  if (!st || !k_slot || !v_slot || !head_stride) return HF_ERR_INVALID_ARG;
  if (!st->win_on || !st->win_ok) return HF_ERR_STATE;
  const hf_config& c = st->cfg;
  hf::BeginPlan p;
  if (n < 1 || n > st->win.win) return HF_ERR_INVALID_ARG;
  if (!hf::plan_begin(st->win, st->next_ev, n, c.max_n_ev, &p)) {
    const int64_t new_hi = st->win.hi + st->win.cur;
    return st->next_ev < st->win.base || st->next_ev > new_hi ? HF_ERR_STATE
                                                              : HF_ERR_INVALID_ARG;
  }
  const size_t row = (size_t)c.head_dim * elem_size(c.dtype);
  const int64_t hs = st->win.cap * c.head_dim;  // elements
  if (p.slide) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool absorbed = false;
    const hf_status r = on_device(st->device, [&]() -> hipError_t {
      hipError_t e = hipSuccess;
      if (p.absorb_n > 0) {
        if (st->spec_n == p.absorb_n && st->spec_lo == st->next_ev) {
          // the previous attend formed these tokens' partial states: reduce them
          st->pend_n = st->spec_n;
          st->spec_n = 0;
          e = flush_pending(st, s);
          if (e != hipSuccess) st->pend_n = 0;
        } else {
          e = enqueue_absorb(st, st->k_ring + p.absorb_row * row,
                             st->v_ring + p.absorb_row * row, p.absorb_n, hs, s);
        }
        absorbed = e == hipSuccess;
      }
      if (e == hipSuccess)
        e = hf::launch_copy_rows_kv(st->k_ring + p.copy_src_row * row,
                                    st->v_ring + p.copy_src_row * row, st->k_ring, st->v_ring,
                                    c.num_heads, (size_t)p.copy_rows * row,
                                    (size_t)hs * elem_size(c.dtype), s);
      return e;
    });
    if (absorbed) st->next_ev += p.absorb_n;
    if (r != HF_OK) {
      st->win_ok = false;  // the ring no longer matches the bookkeeping
      return r;
    }
  }
  hf::apply_begin(&st->win, p, n);
  *k_slot = st->k_ring + p.slot_row * row;
  *v_slot = st->v_ring + p.slot_row * row;
  *head_stride = hs;
  return HF_OK;
}

hf_status hf_window_attend(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                           int32_t top_k, void* out, int64_t out_head_stride, int32_t* sel_out,
                           void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (st->rope.cs) return HF_ERR_UNSUPPORTED;
  if (!st->win_on || !st->win_ok || st->win.cur == 0) return HF_ERR_STATE;
  const hf_config& c = st->cfg;
  if (st->next_ev < st->win.base || st->next_ev > st->win.hi) return HF_ERR_STATE;
  const hf::AttendView v = hf::attend_view(st->win, st->next_ev);
  if (v.ev_n > c.max_n_ev) return HF_ERR_INVALID_ARG;
  const size_t row = (size_t)c.head_dim * elem_size(c.dtype);
  const int64_t hs = st->win.cap * c.head_dim;
  const void* k_win = st->k_ring + v.win_row * row;
  const void* v_win = st->v_ring + v.win_row * row;
  const hf_status e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, v.n_kv, hs,
                                       top_k, out, out_head_stride, sel_out);
  if (e != HF_OK) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* k_ev = st->k_ring + v.ev_row * row;
  const void* v_ev = st->v_ring + v.ev_row * row;
  // Key sums are cached where the window holds whole 8-token groups; only groups
  // of past chunks stay cached, since the current chunk's keys may still change.
  const bool cached = check_window(v.ws, v.n_kv) == HF_OK;
  const hf::KeyCache kc = key_cache(st, v.ws);
  // The tokens that leave the window at the next chunk if it has this chunk's size. If
  // they all belong to past chunks (whose K and V no longer change), their partial
  // states are formed in this call's attention launch; the next absorb uses them if it
  // absorbs exactly these tokens.
  const int64_t end = st->win.hi + st->win.cur;
  const int64_t nx_lo = v.ws;
  const int64_t nx_hi = hf::window_start(end + st->win.cur, st->win.win, v.ws);
  const int64_t nx_n = nx_hi - nx_lo;
  const bool spec_have = nx_n > 0 && st->spec_n == nx_n && st->spec_lo == nx_lo;
  const bool form = n_q > 0 && nx_n > 0 && nx_n <= c.max_n_ev && nx_hi <= st->win.hi &&
                    !spec_have;
  const bool spec_hit = v.ev_n > 0 && st->spec_n == v.ev_n && st->spec_lo == st->next_ev;
  bool absorbed = false, formed = false;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    if (spec_hit) {  // reduced as the pending absorb: in the selection launch, or alone
      st->pend_n = st->spec_n;
      st->spec_n = 0;
    }
    if (n_q == 0) {
      hipError_t err = hipSuccess;
      if (v.ev_n > 0) {
        err = spec_hit ? flush_pending(st, s) : enqueue_absorb(st, k_ev, v_ev, v.ev_n, hs, s);
        absorbed = err == hipSuccess;
      }
      return err;
    }
    const FusedAbsorb fa{k_ev, v_ev, v.ev_n, hs};
    const FusedAbsorb nx{st->k_ring + (nx_lo - st->win.base) * row,
                         st->v_ring + (nx_lo - st->win.base) * row, nx_n, hs};
    const hipError_t err =
        enqueue_attend(st, q, n_q, q_head_stride, k_win, v_win, v.n_kv, hs, top_k, out,
                       out_head_stride, sel_out, s, nullptr,
                       v.ev_n > 0 && !spec_hit ? &fa : nullptr, &absorbed,
                       cached ? &kc : nullptr, form ? &nx : nullptr, &formed);
    if (spec_hit) absorbed = st->pend_n == 0;  // the selection launch reduced them
    return err;
  });
  if (spec_hit && st->pend_n != 0) st->pend_n = 0;  // not enqueued: dropped
  if (cached && n_q > 0) {
    const int64_t past = st->win.hi / 8;  // whole groups of past chunks
    if (st->kc_hi > past) st->kc_hi = past;
    if (st->kc_lo > st->kc_hi) st->kc_lo = st->kc_hi;
  }
  if (absorbed) st->next_ev += v.ev_n;
  if (formed) {
    st->spec_lo = nx_lo;
    st->spec_n = nx_n;
  }
  return r;
}

hf_status hf_window_range(const hf_state* st, int64_t* first, int64_t* count) {
  if (!st || !first || !count) return HF_ERR_INVALID_ARG;
  if (!st->win_on) return HF_ERR_STATE;
  const hf::AttendView v = hf::attend_view(st->win, st->next_ev);
  *first = v.ws;
  *count = v.n_kv;
  return HF_OK;
}

hf_status hf_key_cache_reset(hf_state* st) {
  if (!st) return HF_ERR_INVALID_ARG;
  st->kc_lo = st->kc_hi = 0;
  return HF_OK;
}

hf_status hf_block_scores(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                          const void* k_win, int64_t n_kv, int64_t kv_head_stride,
                          float* scores_out, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  const hf_config& c = st->cfg;
  hf_status e = check_attend(st, q, n_q, q_head_stride, k_win, n_kv, kv_head_stride);
  if (e == HF_OK) e = check_rope_shapes(st, n_q, n_kv);
  if (e != HF_OK) return e;
  if (!scores_out || (reinterpret_cast<uintptr_t>(scores_out) & 3u)) return HF_ERR_INVALID_ARG;
  if (n_q == 0) return HF_OK;
  const int nqb = (int)ceil_div(n_q, c.block_size);
  const int nkb = (int)ceil_div(n_kv, c.block_size);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() {
    hf::Rope rope = st->rope;
    if (rope.cs) rope.q_row0 = n_kv - n_q;
    hipError_t r = hf::launch_block_pool(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q,
                                         q_head_stride, k_win, n_kv, kv_head_stride,
                                         st->pooled_q, st->pooled_k, st->nqb_cap, st->nkb_cap, s,
                                         hf::KeyCache(), rope);
    if (r == hipSuccess)
      r = hf::launch_score_select(c.num_heads, c.head_dim, nqb, nkb, st->nqb_cap, st->nkb_cap,
                                  st->pooled_q, st->pooled_k, st->scale, 1, nullptr, scores_out,
                                  s);
    return r;
  });
}

// Backward workspace: per-row statistics, then the inverse selection index.
struct BwdLayout {
  size_t rowstats, inv_cnt, inv_list, state_part, total;
};

static BwdLayout bwd_layout(const hf_config* c) {
  const size_t H = (size_t)c->num_heads;
  const size_t nqb = (size_t)ceil_div(c->max_n_q, c->block_size);
  const size_t nkb = (size_t)ceil_div(c->max_n_kv, c->block_size);
  BwdLayout L;
  size_t off = 0;
  L.rowstats = off;
  off += round_up(H * (size_t)c->max_n_q * 4 * 4);
  L.inv_cnt = off;
  off += round_up(H * nkb * 4);
  L.inv_list = off;
  off += round_up(H * nkb * nqb * 4);
  L.state_part = off;  // bf16 states: partial dS and dz per 256-row chunk
  if (c->dtype == HF_BF16)
    off += round_up(H * (size_t)ceil_div(c->max_n_q, hf::kBwdStateChunk) *
                    ((size_t)c->head_dim * c->head_dim + c->head_dim) * 4);
  L.total = off;
  return L;
}

static hf_status check_f32_out(const float* p, int64_t n, int64_t head_stride, int d) {
  if (!p || !aligned16(p)) return HF_ERR_INVALID_ARG;
  if (head_stride < n * d || head_stride % 4 != 0) return HF_ERR_INVALID_ARG;
  return HF_OK;
}

size_t hf_backward_workspace_bytes(const hf_config* cfg) {
  if (check_config(cfg) != HF_OK) return 0;
  return bwd_layout(cfg).total;
}

hf_status hf_attend_backward(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                             const void* k_win, const void* v_win, int64_t n_kv,
                             int64_t kv_head_stride, const int32_t* sel, int32_t top_k,
                             const void* dout, int64_t dout_head_stride, float* dq,
                             int64_t dq_head_stride, float* dk_win, float* dv_win,
                             int64_t dkv_head_stride, float* dS, float* dz, void* bwd_ws,
                             size_t bwd_ws_bytes, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (st->rope.cs) return HF_ERR_UNSUPPORTED;  // the backward has no rotation
  const hf_config& c = st->cfg;
  if (n_q < 1) return HF_ERR_INVALID_ARG;
  hf_status e = check_attend_all(st, q, n_q, q_head_stride, k_win, v_win, n_kv, kv_head_stride,
                                 top_k, dout, dout_head_stride, nullptr);
  if (e == HF_OK) e = check_f32_out(dq, n_q, dq_head_stride, c.head_dim);
  if (e == HF_OK) e = check_f32_out(dk_win, n_kv, dkv_head_stride, c.head_dim);
  if (e == HF_OK) e = check_f32_out(dv_win, n_kv, dkv_head_stride, c.head_dim);
  if (e == HF_OK) e = check_f32_out(dS, 1, (int64_t)c.head_dim * c.head_dim, c.head_dim);
  if (e == HF_OK) e = check_f32_out(dz, 1, c.head_dim, c.head_dim);
  if (e != HF_OK) return e;
  if (!sel || (reinterpret_cast<uintptr_t>(sel) & 3u)) return HF_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(&c);
  if (!bwd_ws || !aligned16(bwd_ws) || bwd_ws_bytes < L.total) return HF_ERR_INVALID_ARG;
  char* w = static_cast<char*>(bwd_ws);
  hf::BwdArgs a;
  a.heads = c.num_heads;
  a.q = q;
  a.n_q = n_q;
  a.q_hs = q_head_stride;
  a.k = k_win;
  a.v = v_win;
  a.n_kv = n_kv;
  a.kv_hs = kv_head_stride;
  a.sel = sel;
  a.top_k = top_k;
  a.S = st->S;
  a.z = st->z;
  a.eps = c.eps;
  a.scale = st->scale;
  a.dout = dout;
  a.do_hs = dout_head_stride;
  a.dq = dq;
  a.dq_hs = dq_head_stride;
  a.dk = dk_win;
  a.dv = dv_win;
  a.dkv_hs = dkv_head_stride;
  a.dS = dS;
  a.dz = dz;
  a.rowstats = reinterpret_cast<float*>(w + L.rowstats);
  a.nq_cap = c.max_n_q;
  a.inv_cnt = reinterpret_cast<int32_t*>(w + L.inv_cnt);
  a.inv_list = reinterpret_cast<int32_t*>(w + L.inv_list);
  a.state_part = reinterpret_cast<float*>(w + L.state_part);
  a.s_split = st->s_split;
  a.nqb_cap = st->nqb_cap;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() {
    hipError_t r = flush_pending(st, s);  // the backward reads S and z
    for (int stage = 0; stage < 4 && r == hipSuccess; ++stage)
      r = timed(st, HF_KERNEL_BWD_INDEX + stage, s, [&]() {
        return hf::launch_attend_backward(c.dtype, c.head_dim, c.block_size, a, stage, s);
      });
    return r;
  });
}

hf_status hf_absorb_backward(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                             int64_t ev_head_stride, const float* dS, const float* dz,
                             float* dk_ev, float* dv_ev, int64_t dev_head_stride, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  const hf_config& c = st->cfg;
  if (n_ev < 0 || n_ev > c.max_n_ev) return HF_ERR_INVALID_ARG;
  if (n_ev == 0) return HF_OK;
  hf_status e = check_tensor(k_ev, n_ev, ev_head_stride, c);
  if (e == HF_OK) e = check_tensor(v_ev, n_ev, ev_head_stride, c);
  if (e == HF_OK) e = check_f32_out(dk_ev, n_ev, dev_head_stride, c.head_dim);
  if (e == HF_OK) e = check_f32_out(dv_ev, n_ev, dev_head_stride, c.head_dim);
  if (e != HF_OK) return e;
  if (!dS || !dz || !aligned16(dS) || !aligned16(dz)) return HF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() {
    return timed(st, HF_KERNEL_ABSORB_BWD, s, [&]() {
      return hf::launch_absorb_backward(c.dtype, c.num_heads, c.head_dim, k_ev, v_ev, n_ev,
                                        ev_head_stride, dS, dz, dk_ev, dv_ev, dev_head_stride, s);
    });
  });
}

hf_status hf_attend_ragged(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                           const void* k_flat, const void* v_flat, const int64_t* kv_offsets,
                           const int32_t* top_k, void* out, int64_t out_head_stride,
                           int32_t* sel_out, void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  const hf_config& c = st->cfg;
  if (c.num_heads > hf::kRaggedMaxHeads) return HF_ERR_UNSUPPORTED;
  if (st->rope.cs) return HF_ERR_UNSUPPORTED;  // positions per head are not modelled
  if (!kv_offsets || !top_k || n_q < 0 || n_q > c.max_n_q) return HF_ERR_INVALID_ARG;
  hf::Ragged rg;
  rg.on = 1;
  rg.off[0] = 0;
  rg.kb0[0] = 0;
  int64_t n_min = INT64_MAX;
  int32_t k_max = 0, nkb_max = 0;
  for (int h = 0; h < c.num_heads; ++h) {
    const int64_t a = kv_offsets[h], b = kv_offsets[h + 1];
    if (a < 0 || b <= a || b - a > c.max_n_kv || b > INT32_MAX) return HF_ERR_INVALID_ARG;
    const int32_t nkb = (int32_t)ceil_div(b - a, c.block_size);
    if (top_k[h] < 1 || top_k[h] > nkb || top_k[h] > c.max_top_k) return HF_ERR_INVALID_ARG;
    rg.off[h] = (int32_t)a;
    rg.off[h + 1] = (int32_t)b;
    rg.top_k[h] = top_k[h];
    rg.kb0[h + 1] = rg.kb0[h] + nkb;
    if (b - a < n_min) n_min = b - a;
    if (top_k[h] > k_max) k_max = top_k[h];
    if (nkb > nkb_max) nkb_max = nkb;
  }
  if (!k_flat || !v_flat || !aligned16(k_flat) || !aligned16(v_flat)) return HF_ERR_INVALID_ARG;
  hf_status e = n_q > 0 ? check_tensor(q, n_q, q_head_stride, c) : HF_OK;
  if (e == HF_OK && n_q > 0) e = check_tensor(out, n_q, out_head_stride, c);
  if (e != HF_OK) return e;
  if (sel_out && (reinterpret_cast<uintptr_t>(sel_out) & 3u)) return HF_ERR_INVALID_ARG;
  if (n_q == 0) return HF_OK;
  const int nqb = (int)ceil_div(n_q, c.block_size);
  int32_t* sel = sel_out ? sel_out : st->sel;
  // The attention's items (head-major) cut into 8 ranges of equal selected-block work,
  // one per XCD: range x ends at the first item whose work prefix reaches (x + 1) / 8.
  {
    int64_t total = 0;
    for (int h = 0; h < c.num_heads; ++h) total += (int64_t)nqb * top_k[h];
    int64_t acc = 0;
    int item = 0, x = 1;
    rg.xcd0[0] = 0;
    for (int h = 0; h < c.num_heads; ++h)
      for (int i = 0; i < nqb; ++i, ++item) {
        acc += top_k[h];
        while (x < 8 && acc * 8 >= total * x) rg.xcd0[x++] = item + 1;
      }
    while (x <= 8) rg.xcd0[x++] = item;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return on_device(st->device, [&]() {
    hipError_t r = flush_pending(st, s);  // the attention reads S and z
    if (r == hipSuccess)
      r = timed(st, HF_KERNEL_BLOCK_POOL, s, [&]() {
      return hf::launch_block_pool(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q,
                                   q_head_stride, k_flat, n_min, 0, st->pooled_q, st->pooled_k,
                                   st->nqb_cap, st->nkb_cap, s, hf::KeyCache(), hf::Rope(), rg);
    });
    if (r == hipSuccess)
      r = timed(st, HF_KERNEL_SCORE_SELECT, s, [&]() {
        return hf::launch_score_select(c.num_heads, c.head_dim, nqb, nkb_max, st->nqb_cap,
                                       st->nkb_cap, st->pooled_q, st->pooled_k, st->scale, k_max,
                                       sel, nullptr, s, rg);
      });
    if (r == hipSuccess)
      r = timed(st, HF_KERNEL_SPARSE_SWA, s, [&]() {
        return hf::launch_sparse_swa(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q,
                                     q_head_stride, k_flat, v_flat, n_min, 0, sel, k_max, st->S,
                                     st->s_split, st->z, c.eps, st->scale, out, out_head_stride,
                                     s, hf::Rope(), rg);
      });
    return r;
  });
}

size_t hf_rope_workspace_bytes(const hf_config* cfg, const hf_rope* rope) {
  if (check_config(cfg) != HF_OK || check_rope(*cfg, rope) != HF_OK || rope->rot_dims == 0)
    return 0;
  return rope_layout(*cfg, *rope).total;
}

hf_status hf_set_rope(hf_state* st, const hf_rope* rope, void* workspace, size_t ws_bytes,
                      void* stream) {
  if (!st) return HF_ERR_INVALID_ARG;
  if (!rope || rope->rot_dims == 0) {
    st->rope = hf::Rope();
    st->rope_cfg = hf_rope{};
    return HF_OK;
  }
  const hf_config& c = st->cfg;
  const hf_status e = check_rope(c, rope);
  if (e != HF_OK) return e;
  const RopeLayout L = rope_layout(c, *rope);
  if (!workspace || !aligned16(workspace) || ws_bytes < L.total) return HF_ERR_INVALID_ARG;
  char* w = static_cast<char*>(workspace);
  hf::Rope r;
  r.cs = reinterpret_cast<const float2*>(w + L.table);
  r.half = rope->rot_dims / 2;
  r.tpf = rope->tokens_per_frame;
  r.cap = rope->cap;
  r.k_out = w + L.k_copy;
  r.k_out_hs = c.max_n_kv * c.head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hf_status rs = on_device(st->device, [&]() {
    return hf::launch_rope_table(const_cast<float2*>(r.cs), L.npos, r.half,
                                 (double)rope->theta_base, s);
  });
  if (rs != HF_OK) return rs;
  st->rope = r;
  st->rope_cfg = *rope;
  return HF_OK;
}

hf_status hf_attend_chunk_noalloc(const hf_config* cfg, const float* S, const float* z,
                                  const void* q, int64_t n_q, int64_t q_head_stride,
                                  const void* k_win, const void* v_win, int64_t n_kv,
                                  int64_t kv_head_stride, int32_t top_k, void* out,
                                  int64_t out_head_stride, int32_t* sel_out, void* stream) {
  if (!cfg) return HF_ERR_INVALID_ARG;
  // The call's own sizes stand in for the capacity limits of a state.
  hf_config c = *cfg;
  c.max_n_q = n_q > 0 ? n_q : 1;
  c.max_n_kv = n_kv > 0 ? n_kv : 1;
  c.max_n_ev = 0;
  c.max_top_k = top_k > 0 ? top_k : 1;
  hf_status e = check_config(&c);
  if (e != HF_OK) return e;
  if (n_q < 0 || n_kv < 1) return HF_ERR_INVALID_ARG;
  if (!S || !z || !aligned16(S) || !aligned16(z)) return HF_ERR_INVALID_ARG;
  e = n_q > 0 ? check_tensor(q, n_q, q_head_stride, c) : HF_OK;
  if (e == HF_OK) e = check_tensor(k_win, n_kv, kv_head_stride, c);
  if (e == HF_OK) e = check_tensor(v_win, n_kv, kv_head_stride, c);
  if (e == HF_OK && n_q > 0) e = check_tensor(out, n_q, out_head_stride, c);
  if (e != HF_OK) return e;
  const int64_t nkb = ceil_div(n_kv, c.block_size);
  if (top_k < 1 || top_k > nkb) return HF_ERR_INVALID_ARG;
  if (sel_out && (reinterpret_cast<uintptr_t>(sel_out) & 3u)) return HF_ERR_INVALID_ARG;
  const NoallocLayout L = noalloc_layout(c, n_q, n_kv, top_k);
  if (L.total > HF_NOALLOC_SCRATCH_BYTES) return HF_ERR_INVALID_ARG;
  if (n_q == 0) return HF_OK;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return HF_ERR_HIP;
  char* scratch = noalloc_scratch(device);
  if (!scratch) return HF_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
  const int nqb = (int)ceil_div(n_q, c.block_size);
  float* pooled_q = reinterpret_cast<float*>(scratch + L.pooled_q);
  float* pooled_k = reinterpret_cast<float*>(scratch + L.pooled_k);
  int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(scratch + L.sel);
  uint16_t* s_split = c.dtype == HF_BF16 ? reinterpret_cast<uint16_t*>(scratch + L.s_split) : nullptr;
  // Every scratch byte a kernel reads is written earlier in the same call, so nothing
  // needs clearing; the same kernels as hf_attend_chunk give the same bits.
  hipError_t r = hipSuccess;
  if (s_split) r = hf::launch_split_state(c.num_heads, c.head_dim, S, s_split, s);
  if (r == hipSuccess)
    r = hf::launch_block_pool(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q,
                              q_head_stride, k_win, n_kv, kv_head_stride, pooled_q, pooled_k, nqb,
                              (int)nkb, s);
  if (r == hipSuccess)
    r = hf::launch_score_select(c.num_heads, c.head_dim, nqb, (int)nkb, nqb, (int)nkb, pooled_q,
                                pooled_k, scale, top_k, sel, nullptr, s);
  if (r == hipSuccess)
    r = hf::launch_sparse_swa(c.dtype, c.num_heads, c.head_dim, c.block_size, q, n_q,
                              q_head_stride, k_win, v_win, n_kv, kv_head_stride, sel, top_k, S,
                              s_split, z, c.eps, scale, out, out_head_stride, s);
  return r == hipSuccess ? HF_OK : HF_ERR_HIP;
}

hf_status hf_profile_start(hf_state* st, int32_t max_launches) {
  if (!st || max_launches < 1 || max_launches > (1 << 20)) return HF_ERR_INVALID_ARG;
  prof_release(st);
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    for (int k = 0; k < HF_KERNEL_COUNT; ++k) {
      st->prof_ev[k].resize(2 * (size_t)max_launches, nullptr);
      for (hipEvent_t& e : st->prof_ev[k]) {
        const hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
          e = nullptr;
          return err;
        }
      }
    }
    return hipSuccess;
  });
  if (r != HF_OK) {
    for (int k = 0; k < HF_KERNEL_COUNT; ++k)
      for (hipEvent_t& e : st->prof_ev[k])
        if (e) (void)hipEventDestroy(e);
    for (int k = 0; k < HF_KERNEL_COUNT; ++k) st->prof_ev[k].clear();
    return r;
  }
  st->prof_cap = max_launches;
  st->prof_on = true;
  return HF_OK;
}

hf_status hf_profile_stop(hf_state* st, double* total_ms, int32_t* launches) {
  if (!st || !total_ms || !launches) return HF_ERR_INVALID_ARG;
  const hf_status r = on_device(st->device, [&]() -> hipError_t {
    for (int k = 0; k < HF_KERNEL_COUNT; ++k) {
      double sum = 0.0;
      for (int i = 0; i < st->prof_n[k]; ++i) {
        hipError_t e = hipEventSynchronize(st->prof_ev[k][2 * i + 1]);
        float ms = 0.f;
        if (e == hipSuccess)
          e = hipEventElapsedTime(&ms, st->prof_ev[k][2 * i], st->prof_ev[k][2 * i + 1]);
        if (e != hipSuccess) return e;
        sum += ms;
      }
      total_ms[k] = sum;
      launches[k] = st->prof_n[k];
    }
    return hipSuccess;
  });
  prof_release(st);
  return r;
}

int64_t hf_next_ev_index(const hf_state* st) { return st ? st->next_ev : -1; }

void hf_state_destroy(hf_state* st) {
  if (!st) return;
  prof_release(st);
  int cur = -1;
  const bool switched = hipGetDevice(&cur) == hipSuccess && cur != st->device &&
                        hipSetDevice(st->device) == hipSuccess;
  release_events(st);
  if (switched) (void)hipSetDevice(cur);
  delete st;
}

const char* hf_status_string(hf_status s) {
  switch (s) {
    case HF_OK: return "HF_OK";
    case HF_ERR_INVALID_ARG: return "HF_ERR_INVALID_ARG: invalid argument";
    case HF_ERR_UNSUPPORTED: return "HF_ERR_UNSUPPORTED: head_dim, block_size or dtype not instantiated";
    case HF_ERR_STATE: return "HF_ERR_STATE: eviction index out of sequence";
    case HF_ERR_HIP: return "HF_ERR_HIP: HIP runtime or launch error";
  }
  return "unknown hf_status";
}

}  // extern "C"
