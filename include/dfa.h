/*
 * dfa.h — C ABI of libdfa.so, the MI355X (gfx950) hot path of DistFlashAttn:
 * blockwise exact causal softmax attention over token chunks.
 *
 * Source of the operations: "DISTFLASHATTN: Distributed Memory-efficient
 * Attention for Long-context LLMs Training" (arXiv 2310.03294), as
 * summarised section by section on its paperlayer.ai page.  The paper
 * prints no API; every call below restates one operation that the paper
 * describes, cited by its section / figure / appendix.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layouts (row-major, head_dim contiguous):
 *   Q, O, dO, dQ, O_partial : [batch, len_q,  heads_q,  head_dim]
 *   K, V, dK, dV            : [batch, len_kv, heads_kv, head_dim]
 *   LSE, delta              : [batch, heads_q, len_q]            (float32)
 * Query head h reads key/value head h / (heads_q / heads_kv) (contiguous
 * grouped-query groups).  LSE is the natural-log log-sum-exp of the scaled
 * scores of a row; a row that sees no key has O = 0 and LSE = -inf.
 *
 * Memory: every tensor pointer is DEVICE memory owned by the caller; the
 * library never allocates, frees or retains device memory of its own.
 * Scratch that a call needs beyond its inputs and outputs (the forward's
 * transposed V; the backward's row-split partials) is a caller-owned
 * device workspace named in the descriptor (dfa_attn_desc.workspace /
 * workspace_bytes), sized by dfa_attn_workspace_size.  Descriptors,
 * work-item arrays and the pointer arrays of dfa_lse_merge are HOST memory
 * read during the call only.
 *
 * Asynchrony: work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 * null stream) and the call returns after enqueueing.  No call
 * synchronises the host with the device, allocates or frees memory.
 *
 * Errors: arguments are checked before anything is enqueued; on a non-OK
 * status nothing was enqueued (except DFA_ERR_HIP, where a launch failed)
 * and dfa_last_error() holds a message.  No C++ exception crosses the ABI.
 * The schedules and all argument checks never touch the HIP runtime, so
 * they work on a machine without a GPU.
 *
 * Thread safety: the library keeps no state between calls (apart from the
 * calling thread's last error message, and the per-device scratch of
 * dfa_attn_fwd_partial_noalloc) and every call may be made from any
 * thread.  A call may enqueue several kernels that pass data through its
 * workspace, so calls that share one workspace must be ordered: issued by
 * one thread on one stream, or on streams ordered with events.  Calls with
 * separate workspaces may be issued concurrently from any threads, on one
 * stream or several.
 */
#ifndef DFA_H
#define DFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFA_OK = 0,
  DFA_ERR_INVALID = 1,      /* malformed argument (null pointer, bad shape) */
  DFA_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented (head_dim, */
                            /* head counts past the 32-bit tile offsets)  */
  DFA_ERR_CAPACITY = 3,     /* output array or workspace too small; the    */
                            /* required size is given                       */
  DFA_ERR_HIP = 4           /* the HIP runtime reported an error            */
} dfa_status;

/* Element type of Q, K, V, dO and the final O.  DFA_BF16: bf16 matrix-core
 * products with fp32 accumulation.  DFA_F32: the exact path; fp32 in and
 * out, scores, exponentials and sums carried in fp64.  Across the ABI a
 * dtype travels as an int32_t holding one of these values (a caller may
 * put any integer there; the library checks it before using it). */
typedef enum { DFA_F32 = 0, DFA_BF16 = 1 } dfa_dtype;

/* One chunk pair of a schedule.  kind: 0 = diagonal pair (q_chunk ==
 * kv_chunk, needs the causal element mask), 1 = full pair (q_chunk >
 * kv_chunk, every score visible), 2 = band pair (q_chunk > kv_chunk, a
 * sliding window hides part of it), 3 = global item (kv_chunk = -1: the
 * query chunk against the replicated global tokens, see
 * dfa_global_window_schedule).  owner = q_chunk: the worker whose query
 * rows these are; owner != worker marks a helper item. */
typedef struct {
  int32_t step, worker, q_chunk, kv_chunk, kind, owner;
} dfa_work_item;

/* Shape and masking of one (query chunk, key/value chunk) pair. */
typedef struct {
  int32_t batch;        /* 0 .. 65535 (0: nothing to do)                  */
  int32_t heads_q;      /* >= 1, a multiple of heads_kv; heads_q *       */
                        /* head_dim < 2^21 (else DFA_ERR_UNSUPPORTED)     */
  int32_t heads_kv;     /* >= 1                                            */
  int32_t head_dim;     /* 64 or 128 (else DFA_ERR_UNSUPPORTED)            */
  int64_t len_q;        /* query rows in the chunk, >= 0, any value        */
  int64_t len_kv;       /* key rows in the chunk,   >= 0, any value        */
  int64_t q_start;      /* global token index of query row 0,  >= 0        */
  int64_t kv_start;     /* global token index of key row 0,    >= 0        */
  int32_t causal;       /* 1: key j visible to query i iff
                               kv_start + j <= q_start + i; 0: all visible */
  float scale;          /* score scale sigma (1/sqrt(head_dim)), finite    */
  int32_t dtype;        /* a dfa_dtype: element type of Q, K, V, O (final)
                           and dO                                          */
  int64_t window;       /* 0: no window.  > 0 (needs causal = 1): local
                           sliding window, key j visible to query i only if
                           (q_start + i) - (kv_start + j) < window, i.e. a
                           query sees itself and the window - 1 tokens
                           before it ([DistFlashAttn App. F])             */
  void* workspace;      /* caller-owned DEVICE scratch for the call, 16-byte
                           aligned, not overlapping any tensor argument;
                           NULL allowed when dfa_attn_workspace_size gives 0 */
  int64_t workspace_bytes; /* its size; a call that needs more returns
                           DFA_ERR_CAPACITY (nothing enqueued)            */
} dfa_attn_desc;

/* The two descriptor calls whose kernels may need scratch. */
typedef enum { DFA_OP_FWD = 0, DFA_OP_BWD = 1 } dfa_op;

/* Device workspace (bytes) that dfa_attn_fwd_partial (op = DFA_OP_FWD) or
 * dfa_attn_bwd (op = DFA_OP_BWD) needs for `desc` (its workspace fields are
 * ignored here).  A pure function of the descriptor's shape, mask and dtype:
 * computed on the host, no HIP call, the same on every device.
 *   forward, bf16: the transposed V (2 * batch * heads_kv * head_dim bytes per
 *     key, keys rounded up to 128); float32: 0.
 *   backward, bf16: the fp32 dK/dV partials of the row split (0 unless a
 *     few key blocks carry most of the pair's query rows, e.g. a short key
 *     range or a window band); float32: 0.
 * Each call writes and reads its workspace in stream order and leaves
 * nothing in it that a later call reads. */
dfa_status dfa_attn_workspace_size(const dfa_attn_desc* desc, int32_t op,
                                   int64_t* bytes);

/* Chunk-pair schedule of P = num_workers workers over P contiguous chunks
 * ([DistFlashAttn §3.2 and Fig. 3; App. B, Figs. 5-6]).
 *   balanced = 0: unbalanced causal ring — at step t worker w >= t does
 *     (w, w - t), the others idle; P steps.
 *   balanced = 1: token-level load balancing — step 0 every worker does
 *     its diagonal; at step t = 1..P/2 worker w >= t does (w, w - t) and a
 *     worker h < t helps owner h + P - t with (h + P - t, h) using its own
 *     key/value chunk, unless P - t == t; 1 + floor(P/2) steps.
 * Writes the P(P+1)/2 items, sorted by (step, worker), to the HOST array
 * `items` of `capacity` entries; *num_items and *num_steps receive the
 * counts.  If capacity is too small: DFA_ERR_CAPACITY with *num_items set
 * to the required count and nothing written.  `items` may be NULL when
 * capacity == 0 (a size query).  num_workers must be in [1, 65536]. */
dfa_status dfa_balanced_schedule(int32_t num_workers, int32_t balanced,
                                 dfa_work_item* items, int64_t capacity,
                                 int64_t* num_items, int32_t* num_steps);

/* Chunk-pair schedule of the local sliding window ([DistFlashAttn App. F]:
 * with a window the work is already nearly even, so each worker keeps its
 * own query chunk and shortens its loop to the key/value chunks that hold
 * keys inside some window of its queries; with window <= chunk_len worker
 * 7 of 8 visits chunks 6 and 7 only).  Worker w does (w, w - t) at step t
 * for every t with (t - 1) * chunk_len + 1 < window (t = 0 always); kind 1
 * when (t + 1) * chunk_len - 1 < window, else 2.  No helper items.  Items
 * sorted by (step, worker); array, capacity and counts as in
 * dfa_balanced_schedule.  num_workers in [1, 65536]; chunk_len and window
 * >= 1. */
dfa_status dfa_window_schedule(int32_t num_workers, int64_t chunk_len,
                               int64_t window, dfa_work_item* items,
                               int64_t capacity, int64_t* num_items,
                               int32_t* num_steps);

/* Sliding window plus global tokens replicated on every worker
 * ([DistFlashAttn App. F]: for global attention the global tokens can be
 * replicated on all workers, so that no step has to gather them).  The
 * global tokens are the first n_global positions of the sequence
 * (1 <= n_global <= chunk_len, all in chunk 0); a query sees its window
 * (as in dfa_window_schedule) and every global token at or before it.
 * Items: the window schedule's, except that a pair over kv chunk 0 covers
 * only that chunk's keys n_global..chunk_len-1 (dropped when n_global =
 * chunk_len), plus one global item per worker at step 0, listed before the
 * worker's other step-0 item: (0, w, w, -1, 3, w), the worker's queries
 * against the n_global global keys (global positions 0..n_global-1, causal,
 * no window), read from the worker's replica.  Every visible (query, key)
 * pair lies in exactly one item's key range.  Array, capacity and counts as
 * in dfa_balanced_schedule. */
dfa_status dfa_global_window_schedule(int32_t num_workers, int64_t chunk_len,
                                      int64_t window, int64_t n_global,
                                      dfa_work_item* items, int64_t capacity,
                                      int64_t* num_items, int32_t* num_steps);

/* Partial attention of one chunk pair: the normalised output and its LSE
 * ([DistFlashAttn App. D]: per pair the forward hands back the output with
 * its log-sum-exp; §3.2: a helper sends exactly this state to the owner).
 *   q [B,len_q,Hq,d], k and v [B,len_kv,Hkv,d] in desc->dtype;
 *   o_part [B,len_q,Hq,d] float32 and lse [B,Hq,len_q] float32 are
 *   overwritten.  Only the causal prefix is computed: key tiles entirely
 *   after a query tile's last row are skipped (§2, §3.2), and with a
 *   window so are key tiles entirely outside every window of the tile's
 *   rows (App. F).  For bf16 inputs the call first writes a transposed copy
 *   of v into desc->workspace (dfa_attn_workspace_size, DFA_OP_FWD). */
dfa_status dfa_attn_fwd_partial(const dfa_attn_desc* desc, const void* q,
                                const void* k, const void* v, float* o_part,
                                float* lse, void* hip_stream);

/* The forward of dfa_attn_fwd_partial for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, but the
 * transposed V lives in a fixed array of the library's own device memory
 * (64 MiB per device, loaded with the library's code, kept until the
 * process ends; its address is resolved on the first call on each device)
 * and desc->workspace is ignored.  The call allocates and frees nothing.
 * A pair whose transposed V exceeds 64 MiB (dfa_attn_workspace_size,
 * DFA_OP_FWD) returns DFA_ERR_CAPACITY.  Every call on a device shares that
 * device's array: calls that overlap on one device (different streams, or
 * host threads interleaving on one stream) race; the array needs no
 * clearing (each call writes all of the part it reads). */
dfa_status dfa_attn_fwd_partial_noalloc(const dfa_attn_desc* desc,
                                        const void* q, const void* k,
                                        const void* v, float* o_part,
                                        float* lse, void* hip_stream);

/* LSE merge of n partial states of the same query rows over disjoint key
 * sets ([DistFlashAttn §3.2, Fig. 3]: the owner rescales the partials it
 * receives with their softmax statistics):
 *   M = max_r LSE_r;  LSE = M + ln sum_r exp(LSE_r - M);
 *   O = sum_r exp(LSE_r - LSE) * O_r,   in ascending r, float32 math;
 *   rows with every LSE_r = -inf give O = 0, LSE = -inf.
 * o_parts / lse_parts: HOST arrays of n DEVICE pointers to float32
 * [batch,len_q,heads,head_dim] / [batch,heads,len_q].  o_out is written in
 * out_dtype (a dfa_dtype), lse_out in float32.  o_out may alias o_parts[0] only when
 * out_dtype == DFA_F32 (each element is read before it is written);
 * lse_out may alias lse_parts[0].  1 <= n <= 64. */
dfa_status dfa_lse_merge(int32_t n, const float* const* o_parts,
                         const float* const* lse_parts, int32_t batch,
                         int32_t heads, int64_t len_q, int32_t head_dim,
                         int32_t out_dtype, void* o_out, float* lse_out,
                         void* hip_stream);

/* Backward of one chunk pair from the SAVED final output and LSE; the
 * forward is never recomputed ([DistFlashAttn §3.3]: checkpointing the
 * FlashAttention output lets its backward reuse it, so the forward runs
 * once).  With P = exp(sigma*QK^T - LSE) on the visible scores:
 *   delta = rowsum(dO * O)                   (computed iff compute_delta)
 *   dS    = P * (dO V^T - delta)
 *   dq   += sigma * dS K        [B,len_q, Hq, d]  float32
 *   dk   += sigma * dS^T Q      [B,len_kv,Hkv,d]  float32, summed over the
 *   dv   += P^T dO              [B,len_kv,Hkv,d]  float32  query-head group
 * o and d_o are [B,len_q,Hq,d] in desc->dtype; lse is the final (merged)
 * [B,Hq,len_q].  delta [B,Hq,len_q] float32 is written when compute_delta
 * is 1 and read otherwise (pass 1 on the first pair of a query chunk and 0
 * on its other pairs).  dq, dk, dv accumulate (+=): the caller zeroes them
 * once and sums over pairs (App. D: the backward returns gradient partials
 * to their owners).  Each call is deterministic.  When few key blocks carry
 * most of the pair's rows (a short key range against a long query chunk, a
 * window band) the dK/dV part splits each block's rows over several
 * workgroups and sums their partials in a fixed order in desc->workspace
 * (dfa_attn_workspace_size, DFA_OP_BWD).  delta is computed whenever
 * compute_delta is 1 and the pair has query rows, also when len_kv is 0. */
dfa_status dfa_attn_bwd(const dfa_attn_desc* desc, const void* q,
                        const void* k, const void* v, const void* o,
                        const float* lse, const void* d_o, float* delta,
                        int32_t compute_delta, float* dq, float* dk,
                        float* dv, void* hip_stream);

/* Emulated exchange of one step on a single device ([DistFlashAttn §3.2]:
 * the next key/value chunk reaches a worker by peer-to-peer communication
 * and is prefetched on a separate stream while the current pair computes;
 * a helper's partial output and LSE travel back the same way).  Copies
 * `bytes` bytes from device memory src to device memory dst on a DMA
 * engine (hipMemcpyDeviceToDeviceNoCU), so the transfer takes no compute
 * units from the attention kernels, as a link transfer would not.
 * Enqueued on hip_stream; bytes >= 0 (0: nothing); dst and src non-null
 * when bytes > 0 and not overlapping (else DFA_ERR_INVALID). */
dfa_status dfa_chunk_transfer(void* dst, const void* src, int64_t bytes,
                              void* hip_stream);

/* Message of the last non-OK status on the calling thread ("" if none). */
const char* dfa_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t dfa_version(void);

/* ---- test support: not part of the hot path ---------------------------
 * Tile shape (query rows per workgroup tile, keys per key tile) that
 * dfa_attn_fwd_partial uses for this descriptor. */
dfa_status dfa_test_tile_shape(const dfa_attn_desc* desc, int32_t* bm,
                               int32_t* bn);

/* Runs the same forward as dfa_attn_fwd_partial and records, per batch
 * row 0 and query-head tile 0, which (query tile, key tile) pairs the
 * kernel visited: visits [ceil(len_q/bm), ceil(len_kv/bn)] uint8 DEVICE
 * array, caller-zeroed; 1 = visited without the element mask (causal or
 * window), 2 = visited with it, 0 = skipped. */
dfa_status dfa_test_fwd_tile_visits(const dfa_attn_desc* desc, const void* q,
                                    const void* k, const void* v,
                                    float* o_part, float* lse,
                                    uint8_t* visits, void* hip_stream);

/* Runs one of the two kernels that dfa_attn_bwd launches, alone, with the
 * same arguments and delta already computed: part 1 = the key-outer dK/dV
 * kernel (dk, dv +=; dq untouched), part 2 = the query-outer dQ kernel
 * (dq +=; dk, dv untouched).  For timing each kernel on its own. */
dfa_status dfa_test_bwd_part(const dfa_attn_desc* desc, const void* q,
                             const void* k, const void* v, const float* lse,
                             const void* d_o, const float* delta, float* dq,
                             float* dk, float* dv, int32_t part,
                             void* hip_stream);

/* Kernel launches that dfa_test_bwd_part(desc, ..., part, ...) makes for
 * its kernel (part 1: the dK/dV kernel, whose diagonal pairs of whole
 * 256-key blocks run as two row-band launches; part 2: the dQ
 * kernel, one launch), written to *launches; 0 for a pair without query
 * rows or keys.  Host arithmetic only (no HIP call): a per-launch time is
 * a call's time divided by this count. */
dfa_status dfa_test_bwd_launches(const dfa_attn_desc* desc, int32_t part,
                                 int32_t* launches);

/* Order in which the bf16 kernels hand out a pair's work, so that the
 * longest workgroups start first: *rows_first_to_last = 1 when the forward
 * and dQ take query-row tiles first to last (the pair's first row sees more
 * keys than its last, as in a band pair whose sliding window leaves the key
 * chunk behind the later rows), 0 for last to first; *keys_last_to_first = 1
 * when dK/dV takes its 256-key blocks last to first (its last block has more
 * query-row steps than its first), 0 for first to last.  The order changes no
 * result.  Host arithmetic only (no HIP call); DFA_ERR_INVALID for a bad
 * descriptor or a null output pointer. */
dfa_status dfa_test_work_order(const dfa_attn_desc* desc, int32_t* rows_first_to_last,
                               int32_t* keys_last_to_first);


#ifdef __cplusplus
}
#endif

#endif /* DFA_H */
