/*
 * hf.h -- C ABI of the MI355X (gfx950) hybrid-attention library (libhf.so).
 *
 * The library computes the per-chunk hybrid attention of Hybrid Forcing, a
 * streaming video generation method (arXiv 2604.10103). Sources:
 *   [EN]  gist.science English summary, "Long-Horizon Streaming Video Generation
 *         via Hybrid Attention with Decoupled Distillation".
 *   [ES]  gist.science Spanish summary, "Resumen Tecnico: Hybrid Forcing".
 *   [ABS] the authors' abstract on the fugumt.com listing of arXiv 2604.10103v1.
 *
 * Two paths are summed into one output ([ES] 2.A.2, last bullet):
 *   - a linear temporal path: a compact per-head state that incrementally absorbs
 *     the tokens evicted from the sliding window and is read at a cost independent
 *     of the stream length ([ABS]; [EN] 2.A.1 "Linear Temporal Attention");
 *   - a block-sparse sliding-window softmax path that scores key blocks by block
 *     importance and keeps only the top-K blocks per query block ([EN] 2.A.2
 *     "Block-Sparse Sliding Window Attention").
 * The pages do not fix the formulas. This library implements (per head, tau =
 * softmax_scale, phi(x) = x + 1 for x > 0 and exp(x) otherwise):
 *   state   S = sum_n v_n phi(k_n)^T  (d x d, value-major: S[j][i]),
 *           z = sum_n phi(k_n)        (d)
 *   scores  s[i][j] = tau * mean(Q rows of query block i) . mean(K rows of window
 *           block j), fp32; blocks tile the chunk and the window from row 0 with a
 *           ragged last block;
 *   select  per query block, the top_k key blocks by (score desc, index asc),
 *           listed in ascending index order;
 *   output  out_r = sum_{t in selected rows} softmax_t(tau q_r . k_t) v_t
 *                 + S phi(q_r) / (z . phi(q_r) + eps).
 *
 * Layouts. Q, K, V and out are [H][N][d] row-major with d fastest; consecutive
 * heads are `*_head_stride` ELEMENTS apart (so a window can be a pointer offset
 * into a longer sequence buffer). Element type: bf16 (HF_BF16) or fp32 (HF_F32),
 * fixed per state. S is [H][d][d] fp32 and z is [H][d] fp32, dense.
 *
 * Ownership. The caller allocates and owns all device memory (Q, K, V, out, S, z,
 * sel_out and the workspace) and keeps it alive until the enqueued work is done.
 * The library allocates only the small host-side handle (and two HIP events),
 * freed by hf_state_destroy. It never allocates device memory. For bf16 states the
 * workspace also holds a derived copy of S (its bf16 hi/lo split) that the
 * library refreshes whenever it updates S, so after hf_state_init S and z must be
 * changed only through the library (to load other values, create a new handle).
 *
 * Asynchrony. Calls validate on the host, enqueue on `stream` (a hipStream_t;
 * NULL = the default stream) and return without synchronising. Device faults
 * surface at the caller's next synchronisation.
 *
 * Graphs. Every call enqueues kernel launches only (no memset, allocation or
 * synchronisation), so hf_attend_chunk and hf_block_scores can be captured into a
 * HIP graph and replayed over the same buffers with new contents. The other calls
 * capture as well, but their host-side bookkeeping (eviction index, key-sum cache,
 * managed window) advances once, at capture, not at each replay.
 *
 * Errors. Status codes only: no abort, no exception across the ABI, no logging.
 * On any error nothing is enqueued and the state is unchanged.
 *   HF_ERR_INVALID_ARG  null pointer; negative size; top_k outside [1, ceil(n_kv/B)]
 *                       or above max_top_k; a head stride below n*d or not a multiple
 *                       of 16 bytes; a pointer not 16-byte aligned; a size above the
 *                       max_* limits of the state.
 *   HF_ERR_UNSUPPORTED  head_dim, block_size or dtype outside the instantiated set:
 *                       head_dim in {64, 128}; bf16 with block_size 64; fp32 with
 *                       block_size 16 or 64. Also a configuration whose
 *                       num_heads * (ceil(max_n_q/B) + ceil(max_n_kv/B)) exceeds 2^26
 *                       (the kernels' launch sizes are 32-bit).
 *   HF_ERR_STATE        ev_index differs from the next expected eviction index
 *                       (a gap or a duplicate in the eviction sequence).
 *   HF_ERR_HIP          a HIP runtime call or kernel launch failed.
 *
 * Threading. One handle must not be used from two host threads at once. Handles
 * are independent of each other (one per attention layer). Two calls that use
 * the same workspace must be ordered on one stream.
 */
#ifndef HF_H_
#define HF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HF_OK = 0,
  HF_ERR_INVALID_ARG = 1,
  HF_ERR_UNSUPPORTED = 2,
  HF_ERR_STATE = 3,
  HF_ERR_HIP = 4
} hf_status;

typedef enum { HF_BF16 = 0, HF_F32 = 1 } hf_dtype;

typedef struct {
  int32_t num_heads;   /* H >= 1 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t block_size;  /* B: rows per query/key block (bf16: 64; fp32: 16 or 64) */
  int32_t dtype;       /* hf_dtype of Q, K, V and out; S and z are always fp32 */
  float eps;           /* added once to the linear normaliser; > 0 and finite (1e-6
                          typical): with eps > 0 an empty state (z = 0) reads as an
                          exactly zero linear term */
  float softmax_scale; /* tau; 0 selects 1/sqrt(head_dim) */
  int64_t max_n_q;     /* capacity limits used to size the workspace */
  int64_t max_n_kv;    /* ceil(max_n_kv / B) must be <= 2048 */
  int64_t max_n_ev;
  int32_t max_top_k;
} hf_config;

typedef struct hf_state hf_state; /* opaque host-side handle */

/* Bytes of device workspace a state with this configuration needs (0 on an
 * invalid or unsupported configuration). */
size_t hf_workspace_bytes(const hf_config* cfg);

/* Create a handle over caller-owned S [H][d][d] fp32, z [H][d] fp32 and a
 * workspace of ws_bytes >= hf_workspace_bytes(cfg) bytes (all device memory,
 * 16-byte aligned). zero_fill != 0 enqueues S = 0, z = 0 (an empty state, [EN]
 * 2.A.1); zero_fill == 0 adopts the current contents of S and z (resume from a
 * checkpoint). next_ev_index is the absolute index of the next token to be
 * evicted (0 for a new stream). *out receives the handle. */
hf_status hf_state_init(const hf_config* cfg, float* S, float* z, void* workspace,
                        size_t ws_bytes, int zero_fill, int64_t next_ev_index,
                        void* stream, hf_state** out);

/* Absorb n_ev evicted tokens into the state ([ABS]; [EN] 2.A.1; [ES] 2.A.1):
 * S[h] += V_ev[h]^T phi(K_ev[h]), z[h] += sum_n phi(K_ev[h][n]). k_ev and v_ev are
 * [H][n_ev][d] with head stride ev_head_stride elements. ev_index is the absolute
 * index of the first evicted token and must equal the state's next eviction
 * index (HF_ERR_STATE otherwise); on success the next index advances by n_ev.
 * n_ev == 0 is a valid no-op. The reduction order is fixed, so results are
 * bitwise reproducible on a given device type (the bf16 token split follows the
 * device's compute-unit count). */
hf_status hf_absorb_evicted(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                            int64_t ev_head_stride, int64_t ev_index, void* stream);

/* Hybrid attention of one chunk ([EN] 2.A.1 and 2.A.2; [ES] 2.A.2): q is
 * [H][n_q][d] (head stride q_head_stride), k_win and v_win are the window
 * [H][n_kv][d] (head stride kv_head_stride, shared by K and V), which includes
 * the current chunk; out is [H][n_q][d] (head stride out_head_stride) in the
 * state's element type. top_k key blocks are kept per query block. If sel_out
 * is not NULL it receives the selection, int32 [H][ceil(n_q/B)][top_k], each
 * row ascending. n_q == 0 is a valid no-op. */
hf_status hf_attend_chunk(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                          const void* k_win, const void* v_win, int64_t n_kv,
                          int64_t kv_head_stride, int32_t top_k, void* out,
                          int64_t out_head_stride, int32_t* sel_out, void* stream);

/* hf_absorb_evicted followed by hf_attend_chunk in one call, with the same
 * results bit for bit. Of the chunk's attention only the sparse attention kernel
 * reads S and z. On one stream (side_stream NULL or equal to stream) the absorb
 * shares the chunk's launches: its partial states are formed in the block pooling
 * launch and reduced in the selection launch, so the call takes three launches
 * instead of five. When side_stream is not NULL and differs from stream, the
 * absorb runs on side_stream instead, overlapping the block scoring and selection:
 * it starts after the work already enqueued on stream, and the sparse attention
 * kernel waits for it (two events of the handle). side_stream belongs to the
 * caller and must not carry other work of this handle meanwhile. Either part may
 * be empty (n_ev == 0, n_q == 0). Both parts are validated before anything is
 * enqueued; the eviction index advances once the absorb is enqueued. */
hf_status hf_absorb_and_attend(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                               int64_t ev_head_stride, int64_t ev_index, const void* q,
                               int64_t n_q, int64_t q_head_stride, const void* k_win,
                               const void* v_win, int64_t n_kv, int64_t kv_head_stride,
                               int32_t top_k, void* out, int64_t out_head_stride,
                               int32_t* sel_out, void* stream, void* side_stream);

/* hf_attend_chunk with cached key pooling. win_index is the absolute index, within
 * the stream, of the window's first token (k_win row 0). The key-block means of the
 * block scores ([EN] 2.A.2) are formed from fp32 sums of 8-token groups of K that
 * the state keeps between calls, keyed by absolute token index: the groups that an
 * earlier cached call of this state summed for its window are read from that cache
 * instead of k_win. A window that moves by one chunk per call therefore reads only
 * the chunk's own keys for the pooling; the attention itself still reads k_win and
 * v_win. Results are bit for bit those of hf_attend_chunk (the pooling always adds
 * 8-token groups in the same order). Requirements (HF_ERR_INVALID_ARG otherwise):
 * win_index >= 0, win_index % 8 == 0 and n_kv % 8 == 0. The caller guarantees that
 * the keys of tokens already cached have not changed (a stream's past keys do not),
 * and that cached calls of a handle are ordered on the device (one stream, or
 * synchronised); hf_key_cache_reset forgets the cache. Workspace: the state reserves
 * H x 2^ceil(log2(ceil(max_n_kv / 8))) x d floats for the cache. */
hf_status hf_attend_chunk_cached(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                                 const void* k_win, const void* v_win, int64_t n_kv,
                                 int64_t kv_head_stride, int64_t win_index, int32_t top_k,
                                 void* out, int64_t out_head_stride, int32_t* sel_out,
                                 void* stream);

/* hf_absorb_and_attend on one stream (its three-launch form) with cached key
 * pooling as in hf_attend_chunk_cached: bit for bit the results of
 * hf_absorb_evicted followed by hf_attend_chunk. */
hf_status hf_absorb_and_attend_cached(hf_state* st, const void* k_ev, const void* v_ev,
                                      int64_t n_ev, int64_t ev_head_stride, int64_t ev_index,
                                      const void* q, int64_t n_q, int64_t q_head_stride,
                                      const void* k_win, const void* v_win, int64_t n_kv,
                                      int64_t kv_head_stride, int64_t win_index, int32_t top_k,
                                      void* out, int64_t out_head_stride, int32_t* sel_out,
                                      void* stream);

/* One chunk of a stream with its absorb one call ahead ([EN] 2.A.1 and 2.A.2; [ABS]):
 * the tokens that leave the window at the NEXT chunk (k_next, v_next: [H][n_next][d],
 * head stride next_head_stride, first absolute index next_index) are known a chunk
 * early, so their partial states are formed inside this call's attention launch, by
 * workgroups appended to it that run in the compute-unit slots the attention leaves
 * free (bf16; fp32 states take a launch after the attention), and kept in the
 * workspace as the handle's pending absorb. The next call of this function reduces the
 * pending absorb into S and z in its selection launch, before its attention reads them.
 * So the sequence
 *     hf_absorb_evicted(E0); ahead(chunk 0, E1); ahead(chunk 1, E2); ...
 *     ahead(chunk c, E(c+1)); hf_absorb_flush()
 * gives the outputs, selections, S and z of
 *     hf_absorb_and_attend(E0, chunk 0); hf_absorb_and_attend(E1, chunk 1); ...
 *     hf_absorb_and_attend(E(c+1), empty chunk)
 * bit for bit (the partial states and their reduce are the same kernels' arithmetic in
 * the same order), with one launch of work fewer per chunk on the critical path. The
 * chunk arguments are those of hf_attend_chunk; win_index >= 0 selects the cached key
 * pooling of hf_attend_chunk_cached (same requirements), win_index < 0 none.
 * next_index must equal the state's next eviction index, which advances by n_next
 * once the partial states are enqueued (n_next == 0: nothing becomes pending). Until
 * it is reduced, S and z lack the pending tokens: every other call of the handle that
 * reads or writes S and z (the absorb and attend calls, the managed window, the ragged
 * attention, hf_attend_backward) first enqueues the pending reduce on its own stream,
 * and hf_absorb_flush does only that; a caller that reads S or z itself flushes first.
 * Calls of one handle stay ordered on one stream (the pending partial states live in
 * its workspace). n_q == 0 forms the partial states in a launch of their own. */
hf_status hf_absorb_and_attend_ahead(hf_state* st, const void* q, int64_t n_q,
                                     int64_t q_head_stride, const void* k_win, const void* v_win,
                                     int64_t n_kv, int64_t kv_head_stride, int64_t win_index,
                                     int32_t top_k, void* out, int64_t out_head_stride,
                                     int32_t* sel_out, const void* k_next, const void* v_next,
                                     int64_t n_next, int64_t next_head_stride,
                                     int64_t next_index, void* stream);

/* Reduce the pending absorb of hf_absorb_and_attend_ahead into S and z on `stream`
 * (a no-op when none is pending). */
hf_status hf_absorb_flush(hf_state* st, void* stream);

/* Tokens of the pending absorb (0: none; -1 for a NULL handle). */
int64_t hf_pending_ev(const hf_state* st);

/* Forget the cached key sums of hf_attend_chunk_cached (for example before the
 * handle serves another stream). Host-side only; enqueues nothing. */
hf_status hf_key_cache_reset(hf_state* st);

/* ---- Library-managed window ----------------------------------------------------
 * The state keeps the sliding window itself ([EN] 2.A.2: attention over the latest
 * frames only; [EN] 2.A.1 and [ABS]: what leaves the window is absorbed into the
 * linear state). Its K and V rows live in a caller-owned ring, and each chunk's K
 * and V are written straight into the ring slot the library names. Tokens keep their
 * absolute stream index: the first token of the first chunk after hf_window_attach
 * is hf_next_ev_index(st). The window of a chunk is the last window_tokens tokens up
 * to and including the chunk. */

/* Attach a window of window_tokens tokens (1 <= window_tokens <= max_n_kv) kept in
 * k_ring and v_ring: caller-owned [H][ring_tokens][d] buffers of the state's element
 * type, head stride ring_tokens * d elements, 16-byte aligned, with ring_tokens >=
 * 2 * window_tokens (a larger ring moves the window less often, see
 * hf_window_begin_chunk). The window starts empty. Host only (enqueues nothing);
 * replaces an earlier window and forgets the cached key sums. HF_ERR_UNSUPPORTED for
 * more than 65535 heads. */
hf_status hf_window_attach(hf_state* st, void* k_ring, void* v_ring, int64_t ring_tokens,
                           int64_t window_tokens);

/* Start a chunk of n tokens (1 <= n <= window_tokens). The previous chunk joins the
 * window's past. *k_slot and *v_slot receive the ring rows for the new chunk's K and
 * V ([H][n][d], head stride *head_stride elements); the caller writes them, ordered
 * on the device before hf_window_attend reads them (for example on `stream`). When
 * the chunk does not fit behind the window in the ring, this call first enqueues on
 * `stream` the absorb of the tokens that leave the window and a copy of the rest of
 * the window to the front of the ring (about every (ring_tokens - window_tokens) / n
 * chunks). HF_ERR_INVALID_ARG if more than max_n_ev tokens would wait for the absorb;
 * HF_ERR_STATE without a window, if the eviction index was moved outside the window's
 * tokens (by hf_absorb_evicted), or after a failed copy (HF_ERR_HIP), which leaves the
 * window unusable until it is attached again. */
hf_status hf_window_begin_chunk(hf_state* st, int64_t n, void* stream, void** k_slot,
                                void** v_slot, int64_t* head_stride);

/* Hybrid attention of the current chunk's queries q ([H][n_q][d]) against the window
 * (the current chunk included) and the state, as hf_absorb_and_attend on one stream:
 * tokens that left the window and are not yet absorbed are absorbed first, in the
 * same three launches. The key pooling uses the state's key-sum cache (as
 * hf_attend_chunk_cached) whenever the window starts on an 8-token group and holds
 * whole groups, caching only the past chunks' keys. It may be called several times
 * per chunk (for example once per denoising step, with the slot's K and V rewritten
 * in between); results are bit for bit those of hf_absorb_and_attend over the same
 * window. The tokens that would leave the window at the next chunk if it had this
 * chunk's size are known now; when they all belong to past chunks, their partial
 * states are formed inside this call's attention launch (as hf_absorb_and_attend_ahead
 * does). They are not absorbed yet: the next absorb of exactly those tokens (at the
 * next chunk's hf_window_begin_chunk slide or hf_window_attend) reduces them instead of
 * forming them again, and any call that forms other partial states drops them, so the
 * results never depend on whether the next chunk had that size. HF_ERR_STATE without
 * a window or before the first hf_window_begin_chunk. */
hf_status hf_window_attend(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                           int32_t top_k, void* out, int64_t out_head_stride, int32_t* sel_out,
                           void* stream);

/* The window the next hf_window_attend sees: absolute index of its first token and
 * its length in tokens (HF_ERR_STATE without a window). */
hf_status hf_window_range(const hf_state* st, int64_t* first, int64_t* count);

/* The pooled block importance scores alone ([EN] 2.A.2), the first stage of
 * hf_attend_chunk: scores_out is fp32 [H][ceil(n_q/B)][ceil(n_kv/B)], dense. The
 * same kernels and arithmetic as hf_attend_chunk produce it. */
hf_status hf_block_scores(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                          const void* k_win, int64_t n_kv, int64_t kv_head_stride,
                          float* scores_out, void* stream);

/* ---- Head-aware ragged windows -------------------------------------------------
 * Related work on the pages ("Resumen Tecnico: Pyramid Forcing", 3 "Optimizacion de
 * Calculo de Cache KV Heterogenea"): attention heads keep KV caches of different
 * lengths, stored as flattened sequences with boundary indices, and attention runs
 * over them with no padding. hf_attend_ragged is hf_attend_chunk where head h attends
 * its own window: rows kv_offsets[h] .. kv_offsets[h + 1] of k_flat and v_flat (rows of
 * head_dim elements of the state's type, 16-byte aligned, one flattened sequence:
 * kv_offsets[h + 1] - kv_offsets[h] >= 1 rows, at most max_n_kv, each head's window right
 * after the previous one's, kv_offsets[num_heads] < 2^31), keeping top_k[h] of its own
 * ceil(rows / block_size) key blocks (1 <= top_k[h] <= max_top_k). kv_offsets and top_k
 * are host arrays of num_heads + 1 and num_heads entries, read during the call. q, out
 * and the state are as in hf_attend_chunk (the chunk's queries are the same for every
 * head). sel_out, if not NULL: int32 [H][ceil(n_q / B)][max_h top_k[h]], row (h, i)
 * holding head h's top_k[h] kept blocks, ascending (the rest of the row is not
 * written). HF_ERR_UNSUPPORTED for more than 64 heads or with the rotation of
 * hf_set_rope on. Three launches, as hf_attend_chunk. */
hf_status hf_attend_ragged(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                           const void* k_flat, const void* v_flat, const int64_t* kv_offsets,
                           const int32_t* top_k, void* out, int64_t out_head_stride,
                           int32_t* sel_out, void* stream);

/* ---- Relative temporal rotation (RoPE) -----------------------------------------
 * [EN] 2.C "Stability Enhancements" (Relative RoPE Constraint); [ES] 2.C: the temporal
 * rotary position indices are bounded, the same in training and inference, and
 * positions are relative offsets. The pages give neither the rotated features, the
 * frequencies nor the bound, so all three are parameters. Once set on a state, the
 * softmax path of hf_attend_chunk, hf_absorb_and_attend and hf_block_scores works on
 * rotated queries and keys: the first rot_dims features of each row turn in adjacent
 * pairs (2i, 2i+1) by the angle p * theta_base^(-2i / rot_dims), where p is the row's
 * position: its frame's offset from the window's first frame (frame = window row /
 * tokens_per_frame), capped at cap; the chunk's queries are the window's last n_q
 * rows. The linear state absorbs and reads unrotated features. The rotation is fused
 * into the block pooling launch, which writes the window's rotated keys into the
 * rotation workspace for the attention kernel; the attention kernel rotates the
 * queries itself (to bf16 for bf16 states, rounding to nearest even). */
typedef struct {
  int32_t rot_dims;         /* rotated features: even, 0 <= rot_dims <= head_dim (0: none) */
  float theta_base;         /* > 0 (10000 is the usual value) */
  int64_t tokens_per_frame; /* >= 8 (an 8-row group then spans at most two frames) */
  int32_t cap;              /* >= 0: the largest position index */
} hf_rope;

/* Bytes of the rotation workspace for this configuration and rotation (0 if either
 * is invalid): the angle table, min(cap, ceil(max_n_kv / tokens_per_frame) - 1) + 1
 * positions x rot_dims / 2 pairs x 8 bytes, and the rotated keys, H x max_n_kv x d
 * elements of the state's type, each rounded up to 256 bytes. */
size_t hf_rope_workspace_bytes(const hf_config* cfg, const hf_rope* rope);

/* Turn the rotation on (rope != NULL and rope->rot_dims > 0) or off (rope == NULL or
 * rot_dims == 0; workspace may then be NULL). workspace: caller-owned device memory of
 * at least hf_rope_workspace_bytes bytes, 16-byte aligned, kept alive while the
 * rotation is on. Enqueues the angle table's computation (double precision, rounded
 * to fp32) on stream. While it is on: attend calls need n_kv a multiple of
 * tokens_per_frame and n_q <= n_kv (HF_ERR_INVALID_ARG otherwise); the cached, managed
 * window and backward calls return HF_ERR_UNSUPPORTED. */
hf_status hf_set_rope(hf_state* st, const hf_rope* rope, void* workspace, size_t ws_bytes,
                      void* stream);

/* ---- Backward pass (fixed selection) ------------------------------------------
 * The method is trained through this path ([EN] 2.B-C, decoupled distillation; the
 * state is learnable, [EN] 2.A.1). With L = sum(dout * out) for the output of
 * hf_attend_chunk and the key-block selection of that call held fixed (a discrete
 * choice, with no gradient), per head: the softmax path gives dv_t = sum_r p_rt
 * dout_r, dk_t = tau sum_r dl_rt q_r and dq_r = tau sum_t dl_rt k_t with dl_rt =
 * p_rt (dout_r . v_t - dout_r . o_swa_r); the linear read, with f = phi(q_r), den =
 * z . f + eps, gives dS = sum_r (dout_r / den) f^T, dz = sum_r c_r f with c_r =
 * -(dout_r . S f) / den^2, and dq_r += phi'(q_r) * (S^T dout_r / den + c_r z). All
 * gradients are fp32 and dense per head; every sum runs in a fixed order (bitwise
 * reproducible on a device type). */

/* Bytes of the backward workspace for this configuration (0 if invalid). */
size_t hf_backward_workspace_bytes(const hf_config* cfg);

/* Gradients of one hf_attend_chunk call. q, k_win, v_win, n_q, n_kv, strides and
 * top_k are those of the forward call; sel is its selection (int32
 * [H][ceil(n_q/B)][top_k], as hf_attend_chunk's sel_out returns). Contract: every
 * row of sel is strictly ascending with indices in [0, ceil(n_kv/B)); any such
 * selection is differentiated exactly (the top-K property is not needed). For a row
 * that breaks the contract (unsorted, repeated or out-of-range indices) the
 * gradients are undefined, but the call stays safe: indices are clamped into the
 * window and each key block lists a query block at most once, so nothing is read
 * or written out of bounds. The row contents live in device memory and are not
 * checked on the host. S and z are the state's current ones, i.e. the state must be as at the
 * forward call. dout ([H][n_q][d], element type of the state, head stride
 * dout_head_stride) is the incoming gradient. Outputs, all fp32 and written
 * whole: dq [H][n_q][d] (head stride dq_head_stride), dk_win and dv_win [H][n_kv][d]
 * (head stride dkv_head_stride; rows of unselected key blocks get 0), dS [H][d][d]
 * and dz [H][d] (dense). bwd_ws: caller-owned device memory of at least
 * hf_backward_workspace_bytes bytes, 16-byte aligned. n_q must be >= 1. Five
 * launches on `stream` for bf16 states (dq and dk/dv on MFMA), four for fp32. */
hf_status hf_attend_backward(hf_state* st, const void* q, int64_t n_q, int64_t q_head_stride,
                             const void* k_win, const void* v_win, int64_t n_kv,
                             int64_t kv_head_stride, const int32_t* sel, int32_t top_k,
                             const void* dout, int64_t dout_head_stride, float* dq,
                             int64_t dq_head_stride, float* dk_win, float* dv_win,
                             int64_t dkv_head_stride, float* dS, float* dz, void* bwd_ws,
                             size_t bwd_ws_bytes, void* stream);

/* Gradients through an absorb ([ABS]; [EN] 2.A.1): given dS [H][d][d] and dz [H][d]
 * (fp32, dense) of the state after absorbing k_ev, v_ev ([H][n_ev][d], head stride
 * ev_head_stride), writes dv_ev[n] = dS phi(k_n) and dk_ev[n] = phi'(k_n) * (dS^T v_n
 * + dz) (fp32 [H][n_ev][d], head stride dev_head_stride). The state is only read for
 * its configuration (the eviction index does not move). n_ev == 0 is a no-op. */
hf_status hf_absorb_backward(hf_state* st, const void* k_ev, const void* v_ev, int64_t n_ev,
                             int64_t ev_head_stride, const float* dS, const float* dz,
                             float* dk_ev, float* dv_ev, int64_t dev_head_stride, void* stream);

/* ---- Allocation-free attention ------------------------------------------------
 * For callers that cannot allocate device memory or hand the library a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. hf_attend_chunk_noalloc computes exactly what hf_attend_chunk computes
 * (same kernels, same bits) for a state holding S and z, without a handle: cfg gives
 * num_heads, head_dim, block_size, dtype, eps and softmax_scale (its max_* fields are
 * ignored); S ([H][d][d] fp32) and z ([H][d] fp32) are read only; the other arguments
 * are those of hf_attend_chunk. The intermediates (pooled block means, the selection
 * when sel_out is NULL, and for bf16 the hi/lo split of S) live in a scratch array of
 * HF_NOALLOC_SCRATCH_BYTES that the library keeps in each device's memory for the
 * life of the process; the call allocates nothing and calls no allocating routine.
 * A call needs, rounded up to 256 bytes each, H*ceil(n_q/B)*d*4 + H*ceil(n_kv/B)*d*4
 * + H*ceil(n_q/B)*top_k*4 (+ H*2*d*d*2 for bf16) bytes of it: 2.8 MB at 12 heads,
 * d = 128, 4680 queries, 14040 window tokens and top_k 55. A larger call fails with
 * HF_ERR_INVALID_ARG and enqueues nothing. All calls on one device share that device's
 * scratch and each overwrites it (every byte read is written earlier in the same
 * call, so nothing needs clearing): calls whose work overlaps on one device race, so
 * order them on one stream or synchronise between them. */
#define HF_NOALLOC_SCRATCH_BYTES (8u << 20)
hf_status hf_attend_chunk_noalloc(const hf_config* cfg, const float* S, const float* z,
                                  const void* q, int64_t n_q, int64_t q_head_stride,
                                  const void* k_win, const void* v_win, int64_t n_kv,
                                  int64_t kv_head_stride, int32_t top_k, void* out,
                                  int64_t out_head_stride, int32_t* sel_out, void* stream);

/* Kernels a state launches, for per-kernel timing. */
typedef enum {
  HF_KERNEL_ABSORB = 0,       /* hf_absorb_evicted (both of its launches) */
  HF_KERNEL_BLOCK_POOL = 1,   /* block means of Q and K (first kernel of an attend call;
                                 in a one-stream hf_absorb_and_attend also the absorb's
                                 partial states) */
  HF_KERNEL_SCORE_SELECT = 2, /* block scores + top-K selection (in a one-stream
                                 hf_absorb_and_attend also the absorb's reduce) */
  HF_KERNEL_SPARSE_SWA = 3,   /* block-sparse attention + linear read + sum */
  HF_KERNEL_BWD_INDEX = 4,    /* hf_attend_backward: inverse selection index */
  HF_KERNEL_BWD_DQ = 5,       /* hf_attend_backward: dq and per-row statistics */
  HF_KERNEL_BWD_DKV = 6,      /* hf_attend_backward: dk and dv */
  HF_KERNEL_BWD_STATE = 7,    /* hf_attend_backward: dS and dz */
  HF_KERNEL_ABSORB_BWD = 8,   /* hf_absorb_backward */
  HF_KERNEL_COUNT = 9
} hf_kernel;

/* Profiling aid (not needed for results). From this call on, every kernel the
 * state launches is bracketed by two HIP events recorded on the same stream,
 * for at most max_launches launches per kernel. The events are created here (no
 * device memory is allocated). Restarting discards earlier records. */
hf_status hf_profile_start(hf_state* st, int32_t max_launches);

/* Wait for the recorded events and write, per hf_kernel, the summed kernel time
 * in milliseconds (total_ms[HF_KERNEL_COUNT]) and the number of timed launches
 * (launches[HF_KERNEL_COUNT]); then stop recording and release the events. */
hf_status hf_profile_stop(hf_state* st, double* total_ms, int32_t* launches);

/* Absolute index of the next token the state expects to absorb (-1 if st is NULL). */
int64_t hf_next_ev_index(const hf_state* st);

/* Free the handle (not the caller's device memory). NULL is allowed. */
void hf_state_destroy(hf_state* st);

/* Static description of a status code. */
const char* hf_status_string(hf_status s);

#ifdef __cplusplus
}
#endif
#endif /* HF_H_ */
