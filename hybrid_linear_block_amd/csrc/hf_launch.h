// hf_launch.h -- internal launchers of libhf's gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hf {

// Compute units of the current device (cached per device).
int device_cu_count();

// ---- absorb: S += V^T phi(K), z += sum phi(K) ------------------------------------
constexpr int kAbsorbMaxSplits = 24;
struct AbsorbPlan {
  int tokens_per_split;
  int n_split;
};
// Token split of an absorb of n_ev tokens (dtype 0 = bf16, 1 = fp32); the same for
// every call with the same arguments on the same device.
AbsorbPlan absorb_plan(int dtype, int heads, int d, int64_t n_ev);
// Workgroups of the partial-state pass of that plan.
int absorb_items(int dtype, int heads, int d, const AbsorbPlan& p);
size_t absorb_partial_floats(int heads, int d);
// Two kernels: per-split partial states into `partials`, then an in-order reduction,
// which also refreshes s_split (if not null) from the new S.
hipError_t launch_absorb(int dtype, int heads, int d, const void* k, const void* v, int64_t n_ev,
                         int64_t head_stride, float* S, float* z, float* partials,
                         uint16_t* s_split, hipStream_t stream);
// The two passes of launch_absorb as separate launches: the partial states of n_ev
// tokens, and their reduce into S, z (and s_split) by a later launch.
hipError_t launch_absorb_parts(int dtype, int heads, int d, const void* k, const void* v,
                               int64_t n_ev, int64_t head_stride, float* partials,
                               hipStream_t stream);
hipError_t launch_absorb_reduce(int dtype, int heads, int d, int64_t n_ev, const float* partials,
                                float* S, float* z, uint16_t* s_split, hipStream_t stream);
// s_split[h] = the bf16 hi and lo parts of S[h] ([H][2][d][d]): x ~= hi + lo, hi =
// bf16(x), lo = bf16(x - hi), both rounded to nearest even. The bf16 attention
// epilogue reads S in this form.
hipError_t launch_split_state(int heads, int d, const float* S, uint16_t* s_split,
                              hipStream_t stream);

// ---- block pooling, scoring and top-K selection ----------------------------------
constexpr int kMaxKeyBlocks = 2048;  // key blocks per window (selection LDS budget)
// Cache of 8-row fp32 sums of K rows for the key-block means, kept across calls:
// group g (rows 8g .. 8g+7 of the stream, counted from its first token) lives in
// ring[h][g % cap][0..d). Groups in [lo, hi) are read from the ring; a launch with
// a ring writes every other group of its window there (windows start on a group and
// hold whole groups). ring == nullptr: no cache (every group is summed from K).
struct KeyCache {
  float* ring = nullptr;
  int64_t cap = 1;  // groups per head, a power of two
  int64_t g0 = 0;   // absolute group of window row 0
  int64_t lo = 0, hi = 0;
};
// Relative temporal rotation of the softmax path's queries and keys: the first
// 2 * half features of a row rotate in pairs (2i, 2i+1) by the angle whose cosine
// and sine are cs[p * half + i], p = min(window row / tpf, cap) the row's position.
// Query row n is window row q_row0 + n. The pooling rotates every row it averages
// and writes the window's rotated keys to k_out ([H][n_kv][d], head stride k_out_hs
// elements, the element type of K) for the attention kernel. cs == nullptr: none.
struct Rope {
  const float2* cs = nullptr;
  int half = 0;
  int64_t tpf = 1;
  int cap = 0;
  int64_t q_row0 = 0;
  void* k_out = nullptr;
  int64_t k_out_hs = 0;
};
// Head-aware ragged windows: head h's window is rows off[h] .. off[h + 1] of K and V
// flattened one head after the other (row stride d, no head stride), with its own top_k;
// its key blocks are kb0[h] .. kb0[h + 1] in the order of all heads' blocks. on == false:
// every head has the call's one window shape.
constexpr int kRaggedMaxHeads = 64;
// The attention launch gives XCD x the (head, query block) items xcd0[x] .. xcd0[x + 1]
// of the head-major order, ranges cut so that every XCD gets the same number of
// selected key blocks (a head's items stay together, which keeps its window in that
// XCD's L2).
struct Ragged {
  int32_t on = 0;
  int32_t off[kRaggedMaxHeads + 1];
  int32_t top_k[kRaggedMaxHeads];
  int32_t kb0[kRaggedMaxHeads + 1];
  int32_t xcd0[9];
};
// cs[p * half + i] = (cos, sin) of p * base^(-2i / (2 half)) for p < npos (computed in
// double precision).
hipError_t launch_rope_table(float2* cs, int npos, int half, double theta_base,
                             hipStream_t stream);
// With rg.on, the key part pools every head's own window (n_kv is then the longest).
hipError_t launch_block_pool(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, int64_t n_kv, int64_t kv_hs,
                             float* pooled_q, float* pooled_k, int nqb_cap, int nkb_cap,
                             hipStream_t stream, const KeyCache& kc = KeyCache(),
                             const Rope& rope = Rope(), const Ragged& rg = Ragged());
// The partial-state pass of an absorb of n_ev evicted tokens (as in launch_absorb)
// and launch_block_pool in one launch: the two read and write different buffers
// and are both bound by memory. The absorb is complete once
// launch_select_and_reduce has run its reduce.
hipError_t launch_absorb_and_pool(int dtype, int heads, int d, int block, const void* k_ev,
                                  const void* v_ev, int64_t n_ev, int64_t ev_hs, float* partials,
                                  const void* q, int64_t n_q, int64_t q_hs, const void* k,
                                  int64_t n_kv, int64_t kv_hs, float* pooled_q, float* pooled_k,
                                  int nqb_cap, int nkb_cap, hipStream_t stream,
                                  const KeyCache& kc = KeyCache(), const Rope& rope = Rope());
// With rg.on, head h selects rg.top_k[h] of its own rg.kb0[h + 1] - rg.kb0[h] key blocks
// (nkb is then the largest count and top_k the row stride of sel).
hipError_t launch_score_select(int heads, int d, int nqb, int nkb, int nqb_cap, int nkb_cap,
                               const float* pooled_q, const float* pooled_k, float scale,
                               int top_k, int32_t* sel, float* scores_out, hipStream_t stream,
                               const Ragged& rg = Ragged());
// launch_score_select and, in the same launch, the reduce of the absorb whose
// partial states launch_absorb_and_pool has written (dtype and n_ev as given there).
hipError_t launch_select_and_reduce(int dtype, int heads, int d, int nqb, int nkb, int nqb_cap,
                                    int nkb_cap, const float* pooled_q, const float* pooled_k,
                                    float scale, int top_k, int32_t* sel, const float* partials,
                                    int64_t n_ev, float* S, float* z, uint16_t* s_split,
                                    hipStream_t stream);

// ---- block-sparse softmax attention + linear read ---------------------------------
// Partial states of an absorb (launch_absorb's plan for n_ev tokens) formed by extra
// workgroups appended to the bf16 attention launch, so that they run in the compute
// units' free slots beside it (n_split == 0: none). The reduce is a later launch's.
struct AbsorbAhead {
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t n_ev = 0, hs = 0;
  int tps = 0, n_split = 0;
  float* partials = nullptr;
  int n_attn_wg = 0;  // set by the launcher: workgroups of the attention part
};
// With rope.cs, the queries are rotated in the kernel and the keys are read from
// rope.k_out (head stride rope.k_out_hs), the rotated keys the pooling wrote, instead
// of k; the linear read uses the unrotated queries.
hipError_t launch_sparse_swa(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, const void* v, int64_t n_kv,
                             int64_t kv_hs, const int32_t* sel, int top_k, const float* S,
                             const uint16_t* s_split, const float* z, float eps, float scale,
                             void* out, int64_t out_hs, hipStream_t stream,
                             const Rope& rope = Rope(), const Ragged& rg = Ragged(),
                             const AbsorbAhead& ab = AbsorbAhead());

// ---- backward (fixed selection) ---------------------------------------------------
struct BwdArgs {
  int heads;
  const void* q;
  int64_t n_q, q_hs;
  const void* k;
  const void* v;
  int64_t n_kv, kv_hs;
  const int32_t* sel;
  int top_k;
  const float* S;
  const float* z;
  float eps, scale;
  const void* dout;
  int64_t do_hs;
  float* dq;
  int64_t dq_hs;
  float* dk;
  float* dv;
  int64_t dkv_hs;
  float* dS;
  float* dz;
  float* rowstats;  // [heads][nq_cap][4]: log2-sum-exp2, D, den, c per query row
  int64_t nq_cap;
  int32_t* inv_cnt;   // [heads][nkb]
  int32_t* inv_list;  // [heads][nkb][nqb_cap]
  int nqb_cap;
  float* state_part;  // bf16 states: [heads][ceil(n_q / 256)][d * d + d], partial dS and dz
  const uint16_t* s_split;  // bf16 states: the state's hi/lo split of S ([heads][2][d][d])
};
// Query rows per partial of the bf16 dS / dz kernel (sizes the backward workspace).
constexpr int kBwdStateChunk = 256;
// dq, dk, dv, dS and dz of the hybrid attention (n_q >= 1), stage by stage in order on
// one stream: stage 0 the inverse selection index, 1 dq and the per-row statistics (two
// launches for bf16 states: the MFMA softmax part, then the linear read's part), 2 dk
// and dv, 3 dS and dz.
hipError_t launch_attend_backward(int dtype, int d, int block, const BwdArgs& a, int stage,
                                  hipStream_t s);
// dk_ev and dv_ev of an absorb from dS and dz (n_ev >= 0).
hipError_t launch_absorb_backward(int dtype, int heads, int d, const void* k, const void* v,
                                  int64_t n_ev, int64_t ev_hs, const float* dS, const float* dz,
                                  float* dk, float* dv, int64_t dev_hs, hipStream_t s);

// ---- utilities -------------------------------------------------------------------
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
// Copy bytes_per_head bytes of each of `heads` heads (head_stride_bytes apart in
// both source and destination) for a K and a V tensor at once; multiples of 16
// bytes, 16-byte aligned, source and destination disjoint.
hipError_t launch_copy_rows_kv(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                               int heads, size_t bytes_per_head, size_t head_stride_bytes,
                               hipStream_t stream);

}  // namespace hf
