/*
 * libringattn -- exact ring-ordered attention (forward and backward) for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (sources: the youngju.dev page "Ring Attention 논문 분석", the
 * Ultralytics glossary page "Ring Attention", the GPU MODE lecture 013 notes
 * and the llm-engineer.pages.dev page "Context Parallelism"): a query chunk
 * stays fixed while the key/value chunks are visited one at a time, chunk
 * (i - step) mod N at step `step` for query chunk i.  Per query row the
 * library keeps the running maximum m of the scaled scores, the running sum
 * l of exp(s - m) and the running output o = sum exp(s - m) v, so that the
 * result equals softmax(scale q k^T) v over all visible keys exactly (up to
 * rounding).  Partials over disjoint key sets combine by log-sum-exp.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are [batch, heads, rows, d] with element strides (b, h, s) given
 *   in the descriptor; the stride of the last dimension is 1.  Query head h
 *   reads key/value head h / (hq / hkv).
 * - Scores are s = scale * <q, k>; scale <= 0 in a descriptor selects
 *   1/sqrt(d).  Logarithms and the returned lse are natural.
 * - Running state is fp32: m and l are [B, Hq, Lq] with strides desc.ml
 *   (ml.s must be 1), o is [B, Hq, Lq, d] with strides desc.o.  m is in
 *   score units; o is unnormalized.  An empty row has m = -inf, l = 0, o = 0.
 * - Causal masking is expressed by one integer offset delta per call: key row
 *   k is hidden from query row p (rows counted from the start of the given
 *   buffers) iff causal != 0 and k - p > delta.  delta = 0 is the usual
 *   lower-triangular mask with the diagonal kept.
 * - Device pointers are owned by the caller.  The library never allocates or
 *   frees device memory and never synchronizes: work is enqueued on `stream`
 *   (a hipStream_t; NULL is the default stream) and completes
 *   asynchronously.  Asynchronous faults surface at the caller's next
 *   synchronization.
 * - Arguments are validated on the host before any HIP call; a rejected call
 *   enqueues nothing.  The library keeps no global mutable state except a
 *   thread-local error message, so calls from several threads are safe.
 *   Nothing is printed and nothing aborts.
 * - Supported: in_dtype BF16 with d = 128 (matrix-core path), in_dtype F32
 *   with d in {16, 32, 64, 128}; out_dtype F32 or BF16.  Other combinations
 *   return RA_ERR_UNSUPPORTED.  Device pointers must be 16-byte aligned and
 *   row strides (s) must be multiples of 8 elements for BF16 and of 4 for
 *   F32; the (b) and (h) strides likewise.  The BF16 path addresses one
 *   head's K or V rows with 32-bit byte offsets and walks at most 1024 KV
 *   segments per call (n_chunks for contiguous / striped, 2 n_chunks for
 *   zig-zag): (kv rows - 1) x row stride + 2d must stay below 2^31 bytes, else
 *   RA_ERR_UNSUPPORTED.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 3

/* Largest ra_ring_desc.kv_splits. */
#define RA_MAX_KV_SPLITS 64

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, stride or alignment */
  RA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype / head dim) */
  RA_ERR_WORKSPACE = 3,   /* workspace smaller than ra_ring_workspace_bytes */
  RA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} ra_status;

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* Token layouts of the sequence over the N chunks (L = seq / N):
 * CONTIGUOUS: row p of chunk c is token c*L + p (consecutive chunks, as in the
 *   data collator of the youngju.dev page and the token split of the
 *   "Context Parallelism" page).
 * STRIPED: row p of chunk c is token p*N + c, i.e. token t lives in chunk
 *   t mod N (striped attention, glossary page "Ring Attention" and lecture
 *   013 notes, first remedy for causal imbalance).
 * ZIGZAG: with s = L/2, rows 0..s-1 of chunk c are tokens c*s + p and rows
 *   s..L-1 are tokens (2N-1-c)*s + (p - s): every chunk holds one early and
 *   one late segment ("Context Parallelism" page, causal imbalance; the page
 *   gives no formula, this is the reading taken). */
typedef enum ra_layout { RA_LAYOUT_CONTIGUOUS = 0, RA_LAYOUT_STRIPED = 1, RA_LAYOUT_ZIGZAG = 2 } ra_layout;

/* Classification of a (query segment, KV segment) pair under causal masking
 * (the ring_attention_causal_step listing of the youngju.dev page: skip a
 * block that lies wholly in the future, mask the diagonal block, compute a
 * past block in full). */
typedef enum ra_kind { RA_FULL = 0, RA_MASKED = 1, RA_SKIP = 2 } ra_kind;

typedef void* ra_stream; /* hipStream_t */

typedef struct ra_strides {
  int64_t b, h, s; /* element strides of the batch, head and row dimensions */
} ra_strides;

typedef struct ra_attn_desc {
  int64_t batch;     /* B >= 1 */
  int64_t hq, hkv;   /* query / key-value heads, hq % hkv == 0 */
  int64_t lq, lk;    /* query rows and key rows, >= 1 */
  int64_t d;         /* head dimension of q, k and v */
  int32_t in_dtype;  /* ra_dtype of q, k, v */
  int32_t out_dtype; /* ra_dtype of the normalized output */
  ra_strides q, k, v, out; /* strides of q, k, v, out (elements) */
  ra_strides ml;     /* strides of m, l and lse (fp32); ml.s must be 1 */
  ra_strides o;      /* strides of the running / partial o (fp32) */
  float scale;       /* <= 0: 1/sqrt(d) */
  int32_t reserved;  /* must be 0 */
} ra_attn_desc;

typedef struct ra_ring_desc {
  /* attn.lq == attn.lk == seq / n_chunks (the chunk length L).
   * q and out hold the q_chunk_count query chunks back to back, physical
   * (chunk-major) order: row (c - q_chunk_first) * L + p is row p of chunk c.
   * k and v hold all n_chunks chunks the same way: row c * L + p.
   * lse (optional) is [B, Hq, q_chunk_count * L] with strides attn.ml. */
  ra_attn_desc attn;
  int64_t seq;           /* total tokens S, a multiple of n_chunks */
  int32_t n_chunks;      /* N >= 1 */
  int32_t layout;        /* ra_layout; ZIGZAG needs an even L */
  int32_t causal;        /* 0 or 1 */
  int32_t q_chunk_first; /* first query chunk computed */
  int32_t q_chunk_count; /* number of consecutive query chunks computed */
  int32_t kv_splits;     /* ra_ring_fwd only: 0 or 1 = one workgroup walks all KV
                          * tiles of its query tile; 2 .. RA_MAX_KV_SPLITS = split-KV
                          * (see ra_ring_fwd); ignored by ra_ring_bwd */
} ra_ring_desc;

/* One (query segment, KV segment) pair of the ring schedule. */
typedef struct ra_task {
  int32_t step;     /* ring step t; the KV chunk is (q_chunk - t) mod N */
  int32_t kv_chunk;
  int32_t q_row0, q_len;   /* row range inside the query chunk */
  int32_t kv_row0, kv_len; /* row range inside the KV chunk */
  int64_t delta;    /* causal offset for rows counted from q_row0 / kv_row0 (0 if not causal) */
  int32_t kind;     /* ra_kind (FULL when not causal) */
  int32_t reserved;
} ra_task;

/* ABI version of the loaded library (RA_ABI_VERSION). */
int ra_abi_version(void);

/* Static text for a status code. */
const char* ra_status_str(ra_status status);

/* Text describing the last non-OK status returned on the calling thread
 * (which argument was rejected, or the HIP error string). */
const char* ra_last_error(void);

/* Set the running state to empty: m = -inf, l = 0, o = 0 (the accumulators
 * that ring_attention_forward of the youngju.dev page starts from).
 * Shapes from desc (batch, hq, lq, d); strides desc.ml and desc.o. */
ra_status ra_state_init(const ra_attn_desc* desc, float* m, float* l, float* o, ra_stream stream);

/* Fold one key/value chunk into the running state (m, l, o) of a query
 * block: the online-softmax update of blockwise_attention and
 * ring_attention_forward (youngju.dev page) and of the m / l / o description
 * of the "Context Parallelism" page.  For every query row the new maximum
 * m' = max(m, max_k s), then l = exp(m - m') l + sum_k exp(s - m') and
 * o = exp(m - m') o + sum_k exp(s - m') v_k over the visible keys.
 * q: [B, Hq, lq, d]; k, v: [B, Hkv, lk, d] (desc.in_dtype, strides desc.q/k/v).
 * m, l, o: running state, read and written in place (fp32).
 * causal / causal_delta: see the conventions above.  A row that sees no key
 * is left unchanged, bit for bit; a row whose maximum does not grow gets its
 * m back bit for bit. */
ra_status ra_chunk_fwd(const ra_attn_desc* desc, const void* q, const void* k, const void* v,
                       float* m, float* l, float* o, int64_t causal_delta, int32_t causal,
                       ra_stream stream);

/* Normalize: out = o / l in desc.out_dtype (strides desc.out) and, if lse is
 * not NULL, lse = m + ln l (fp32, strides desc.ml): the final division of
 * blockwise_attention and the log-sum-exp of lecture 013, section 03, which
 * the backward listing of the youngju.dev page consumes.  Rows with l = 0
 * give out = 0 and lse = -inf.  out must not overlap m, l or o. */
ra_status ra_finalize(const ra_attn_desc* desc, const float* m, const float* l, const float* o,
                      void* out, float* lse, ra_stream stream);

/* Combine two normalized partials over disjoint key sets by log-sum-exp
 * associativity (lecture 013 notes, section 03): with M = max(lse_a, lse_b),
 * lse = M + ln(exp(lse_a - M) + exp(lse_b - M)) and
 * o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b.  A partial with lse = -inf
 * contributes nothing.  lse_*: [B, Hq, lq] (strides desc.ml); o_*:
 * [B, Hq, lq, d] fp32 (strides desc.o).  lse_out / o_out may be the same
 * pointers as lse_a / o_a or lse_b / o_b (in-place merge); any other overlap
 * is undefined. */
ra_status ra_merge(const ra_attn_desc* desc, const float* lse_a, const float* o_a,
                   const float* lse_b, const float* o_b, float* lse_out, float* o_out,
                   ra_stream stream);

/* Workspace bytes ra_ring_fwd needs for this descriptor: 0 without split-KV,
 * else kv_splits * B * Hq * (q_chunk_count * L) * (d + 1) fp32 values (the
 * partial o and lse of every KV range). */
size_t ra_ring_workspace_bytes(const ra_ring_desc* desc);

/* The whole ring: for every requested query chunk i, fold in KV chunks
 * (i - t) mod N for t = 0 .. N-1 (the ring order of the glossary page's
 * four-device simulation and of ring_attention_forward), skip chunk-pair
 * segments that are wholly in the future, mask the ones that straddle the
 * diagonal, and finalize.  One fused launch: the state stays on chip from the
 * first step to the last.  out: desc.attn.out_dtype, strides desc.attn.out;
 * lse may be NULL.  Rows that see no key give out = 0, lse = -inf.
 * Split-KV (desc.kv_splits = S > 1; for few query rows, or causal work that
 * differs much between query tiles): the KV tiles one query tile visits, in
 * ring order, are cut into S consecutive ranges of nearly equal tile counts,
 * each walked by its own workgroup into a normalized partial (o_s, lse_s) in
 * the workspace, and a second kernel merges them with the log-sum-exp
 * associativity of the lecture 013 notes (lse = M + ln sum_s e^(lse_s - M), out =
 * sum_s e^(lse_s - lse) o_s, M = max lse_s; the pairwise merge of ra_merge
 * folded over all S at once).  Same result up to rounding.  workspace: device
 * memory of ra_ring_workspace_bytes(desc) bytes, 16-byte aligned, used during
 * the call only (may be NULL when that is 0). */
ra_status ra_ring_fwd(const ra_ring_desc* desc, const void* q, const void* k, const void* v,
                      void* out, float* lse, void* workspace, size_t workspace_bytes,
                      ra_stream stream);

/* One ring step of one query chunk, as a device of the ring runs it when a
 * KV chunk arrives (ring_attention_forward on the youngju.dev page: step t of
 * query chunk i folds in KV chunk j = (i - t) mod N; the glossary page's
 * four-device simulation): skip the segment pairs wholly in the future, mask
 * the ones on the diagonal, fold the rest into the running (m, l, o), which
 * stays in device memory between steps.  Starting from ra_state_init and
 * ending with ra_finalize, the N steps in any order give ra_ring_fwd's result
 * (the order changes rounding only).
 * desc: q_chunk_count must be 1, the query chunk is q_chunk_first; kv_splits
 * is not used.  q: that chunk's rows [B, Hq, L, d] (strides desc.attn.q);
 * k, v: the rows of KV chunk j only, [B, Hkv, L, d] (strides desc.attn.k /
 * desc.attn.v), in the chunk's physical row order; m, l: [B, Hq, L] fp32
 * (strides desc.attn.ml); o: [B, Hq, L, d] fp32 (strides desc.attn.o), all
 * read and overwritten (m natural, relative to which l and o are kept, as
 * ra_chunk_fwd).  A step with nothing visible returns without a launch. */
ra_status ra_ring_step(const ra_ring_desc* desc, int32_t step, const void* q, const void* k, const void* v,
                       float* m, float* l, float* o, ra_stream stream);

/* Host only.  A kv_splits value for ra_ring_fwd on this descriptor: 1 when
 * the query tiles alone give every compute unit two workgroups or more, else
 * enough KV ranges for about four per compute unit (at most
 * RA_MAX_KV_SPLITS, and at most one per 256 keys of the sequence).
 * desc.kv_splits itself is not read. */
ra_status ra_ring_kv_splits_hint(const ra_ring_desc* desc, int32_t* splits);

/* Workspace bytes ra_ring_bwd needs for this descriptor: two fp32 values per
 * (batch, query head, query row) of the requested query chunks. */
size_t ra_ring_bwd_workspace_bytes(const ra_ring_desc* desc);

/* Backward of ra_ring_fwd for the requested query chunks: the steps of
 * ring_attention_backward on the youngju.dev page.  Per query row
 * D = rowsum(dout * out); per visible (query, key) pair P = exp(s - lse) is
 * recomputed from the forward's log-sum-exp, and
 *   dv += P^T dout,  dP = dout v^T,  dS = P (dP - D) scale,
 *   dq += dS k,      dk += dS^T q,
 * visiting the KV chunks in ring order for dq and every requested query row
 * for dk, dv.  With grouped heads dk and dv of a KV head sum the
 * contributions of all its query heads.
 * Inputs (device): q, k, v as for ra_ring_fwd; out (the forward's output,
 * desc.attn.out_dtype, strides desc.attn.out); dout (bf16, strides
 * desc.attn.out, which must then be multiples of 8 elements whatever
 * out_dtype is); lse (natural, fp32, strides desc.attn.ml) as ra_ring_fwd
 * writes it.
 * Outputs (device, fp32, overwritten): dq with the element strides of q;
 * dk and dv with the element strides of k and v, for all n_chunks chunks:
 * the share of the requested query rows (the full gradient when every query
 * chunk is requested; on several devices these shares are what the pages'
 * listing reduces to the owner of each KV chunk).  Keys no requested row
 * sees get 0.
 * workspace: device memory of ra_ring_bwd_workspace_bytes(desc) bytes, 16-byte
 * aligned, used during the call only.
 * Supported: in_dtype BF16 with d = 128 (RA_ERR_UNSUPPORTED otherwise); the
 * limits of ra_ring_fwd apply, and one head's query and dout rows must also
 * span less than 2 GiB.  Three kernels are enqueued on `stream`. */
ra_status ra_ring_bwd(const ra_ring_desc* desc, const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, float* dq, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, ra_stream stream);

/* Largest workspace, in bytes, that ra_ring_bwd_noalloc brings with it: 8
 * bytes per (batch, query head, query row) of the requested query chunks, so
 * at most 2^21 such rows per call. */
#define RA_BWD_NOALLOC_MAX_BYTES (16u << 20)

/* ra_ring_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and results, without the workspace arguments.
 * The workspace is a file-scope device array of RA_BWD_NOALLOC_MAX_BYTES in
 * the library, one copy on each GPU it runs on, held until the process ends;
 * it is looked up once per GPU (the GPU of `stream`, or the current GPU for
 * the NULL stream) and nothing is allocated or freed by the call.  Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other threads) race; serialize them.  Every workspace value a call
 * reads is written earlier in the same call, so nothing needs clearing.
 * A call that needs more than RA_BWD_NOALLOC_MAX_BYTES of workspace returns
 * RA_ERR_UNSUPPORTED (use ra_ring_bwd with a workspace); a failed lookup
 * returns RA_ERR_HIP. */
ra_status ra_ring_bwd_noalloc(const ra_ring_desc* desc, const void* q, const void* k, const void* v,
                              const void* out, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                              ra_stream stream);

/* Host only.  pos[p] = global token position of row p of chunk `chunk`
 * (p = 0 .. seq/n_chunks - 1) under `layout`: the token split of the
 * "Context Parallelism" page (each GPU takes a chunk of consecutive tokens;
 * causal imbalance, where the zig-zag mix of early and late tokens is
 * proposed without a formula) and the striped assignment of the glossary page
 * "Ring Attention" (how it works: tokens spread evenly over the devices); the
 * maps are those of ra_layout above.  pos is host memory of seq / n_chunks
 * entries. */
ra_status ra_layout_positions(int32_t layout, int64_t seq, int32_t n_chunks, int32_t chunk,
                              int64_t* pos);

/* Host only.  The schedule that ra_ring_fwd runs for query chunk q_chunk, in
 * ring order: per step, every (query segment, KV segment) pair with its
 * causal offset and kind (SKIP pairs are listed; ra_ring_fwd does not run
 * them).  The order is the ring order of ring_attention_forward on the
 * youngju.dev page (step t visits KV chunk (q_chunk - t) mod N) and the kinds
 * are the three cases of its ring_attention_causal_step listing (a future
 * block is skipped, the diagonal block is masked, a past block is computed
 * in full).  Writes up to `capacity` entries to the host array `tasks` and the
 * total count to *n_tasks; returns RA_ERR_INVALID_ARG if capacity is too
 * small (n_tasks still receives the count). */
ra_status ra_ring_schedule(const ra_ring_desc* desc, int32_t q_chunk, ra_task* tasks,
                           int32_t capacity, int32_t* n_tasks);

/* Reorder rows between logical token order and the chunk-major physical
 * order of `layout` (a gather or scatter along the row dimension; a bit-exact
 * copy): the split of the sequence over the devices that the data collator of
 * the youngju.dev page (LongContextDataCollator) and the token chunks of the
 * "Context Parallelism" page perform, with the row maps of ra_layout.  src and dst are contiguous [batch, heads, seq, d] of `dtype` and
 * must not overlap.  to_chunked != 0: dst row c*L + p = src row pos(c, p);
 * to_chunked == 0: the inverse. */
ra_status ra_permute(int32_t layout, int32_t to_chunked, int64_t batch, int64_t heads, int64_t seq,
                     int32_t n_chunks, int64_t d, int32_t dtype, const void* src, void* dst,
                     ra_stream stream);

/* ra_permute on strided tensors: src and dst are [batch, heads, seq, d] of
 * `dtype` with element strides (sb, sh, ss) each and a contiguous last
 * dimension, so a [batch, seq, heads, d] buffer (the layout of the JAX ring
 * listing on the youngju.dev page) is read or written in place of a
 * transposed copy.  Strides must not be negative and pointers must be
 * aligned to the element (else RA_ERR_INVALID_ARG).  The rows src reads and
 * the rows dst writes must not overlap (not checked).  Same row maps and
 * bit-exact copy as ra_permute. */
ra_status ra_permute_strided(int32_t layout, int32_t to_chunked, int64_t batch, int64_t heads, int64_t seq,
                             int32_t n_chunks, int64_t d, int32_t dtype, const void* src, int64_t src_sb,
                             int64_t src_sh, int64_t src_ss, void* dst, int64_t dst_sb, int64_t dst_sh,
                             int64_t dst_ss, ra_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
