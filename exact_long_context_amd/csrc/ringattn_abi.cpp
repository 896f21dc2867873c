// The C ABI of libringattn: argument validation (on the host, before any HIP
// call), the host-side schedule and layout queries, and the launch planning
// of the kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/ringattn.h"
#include "kernels.h"
#include "schedule.h"

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ra_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RA_OK;
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t I32_MAX = 2147483647;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }

ra_status check_strides(const char* name, const ra_strides& s, int32_t dtype) {
  const int64_t unit = 16 / elem_bytes(dtype);
  if (s.b < 0 || s.h < 0 || s.s < 0) return fail(RA_ERR_INVALID_ARG, "%s: negative stride", name);
  if (s.b % unit || s.h % unit || s.s % unit)
    return fail(RA_ERR_INVALID_ARG, "%s: strides must be multiples of %lld elements", name, (long long)unit);
  return RA_OK;
}

// Shape, dtype and stride checks common to every entry point that takes an
// attention descriptor.
ra_status check_attn(const ra_attn_desc* d) {
  if (d == nullptr) return fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->reserved != 0) return fail(RA_ERR_INVALID_ARG, "reserved field must be 0");
  if (d->batch < 1 || d->hq < 1 || d->hkv < 1 || d->lq < 1 || d->lk < 1 || d->d < 1)
    return fail(RA_ERR_INVALID_ARG, "batch, heads, rows and d must be >= 1");
  if (d->hq % d->hkv) return fail(RA_ERR_INVALID_ARG, "hq (%lld) is not a multiple of hkv (%lld)",
                                  (long long)d->hq, (long long)d->hkv);
  if (d->lq > I32_MAX || d->lk > I32_MAX || d->batch * d->hq > I32_MAX)
    return fail(RA_ERR_INVALID_ARG, "rows or batch*heads exceed 2^31-1");
  if (d->in_dtype != RA_F32 && d->in_dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "unknown in_dtype");
  if (d->out_dtype != RA_F32 && d->out_dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "unknown out_dtype");
  if (!(d->scale <= 0.f || std::isfinite(d->scale))) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  if (d->in_dtype == RA_BF16 && d->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "bf16 inputs need d = 128 (got %lld)", (long long)d->d);
  if (d->in_dtype == RA_F32 && d->d != 16 && d->d != 32 && d->d != 64 && d->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "fp32 inputs need d in {16, 32, 64, 128} (got %lld)", (long long)d->d);
  ra_status st;
  if ((st = check_strides("q", d->q, d->in_dtype)) != RA_OK) return st;
  if ((st = check_strides("k", d->k, d->in_dtype)) != RA_OK) return st;
  if ((st = check_strides("v", d->v, d->in_dtype)) != RA_OK) return st;
  if ((st = check_strides("out", d->out, d->out_dtype)) != RA_OK) return st;
  if ((st = check_strides("o", d->o, RA_F32)) != RA_OK) return st;
  if (d->ml.s != 1) return fail(RA_ERR_INVALID_ARG, "ml.s must be 1");
  if (d->ml.b < 0 || d->ml.h < 0) return fail(RA_ERR_INVALID_ARG, "ml: negative stride");
  return RA_OK;
}

// The row kernels give every row d/8 lanes; d is one of 16..128 here.
ra::RowsArgs rows_args(const ra_attn_desc* d) {
  ra::RowsArgs g;
  g.batch = (int32_t)d->batch;
  g.heads = (int32_t)d->hq;
  g.rows = (int32_t)d->lq;
  g.d = (int32_t)d->d;
  g.ml_sb = d->ml.b; g.ml_sh = d->ml.h;
  g.o_sb = d->o.b; g.o_sh = d->o.h; g.o_ss = d->o.s;
  g.out_sb = d->out.b; g.out_sh = d->out.h; g.out_ss = d->out.s;
  return g;
}

float log2_scale(const ra_attn_desc* d) {
  const double sc = d->scale > 0.f ? (double)d->scale : 1.0 / std::sqrt((double)d->d);
  return (float)(sc * 1.4426950408889634074);
}

void fill_common(ra::FwdArgs& a, const ra_attn_desc* d, const void* q, const void* k, const void* v) {
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v;
  a.q_sb = d->q.b; a.q_sh = d->q.h; a.q_ss = d->q.s;
  a.k_sb = d->k.b; a.k_sh = d->k.h; a.k_ss = d->k.s;
  a.v_sb = d->v.b; a.v_sh = d->v.h; a.v_ss = d->v.s;
  a.ml_sb = d->ml.b; a.ml_sh = d->ml.h;
  a.o_sb = d->o.b; a.o_sh = d->o.h; a.o_ss = d->o.s;
  a.out_sb = d->out.b; a.out_sh = d->out.h; a.out_ss = d->out.s;
  a.out_bf16 = d->out_dtype == RA_BF16;
  a.batch = (int32_t)d->batch;
  a.hq = (int32_t)d->hq;
  a.hkv = (int32_t)d->hkv;
  a.d = (int32_t)d->d;
  a.scale_log2 = log2_scale(d);
  a.kv_splits = 1;
}

// Work decomposition.  bf16: 8 waves of 32 rows per workgroup; the waves are
// query heads of one KV head when the group size allows (GQA shares every K/V
// tile over the heads), else consecutive row blocks of one head.  fp32: 4
// waves of 32 rows of one head.
ra_status plan_launch(ra::FwdArgs& a, bool bf16, int64_t seg_len, int32_t nseg_q, int32_t q_count) {
  const int32_t G = a.hq / a.hkv;
  if (bf16) {
    // 8 waves of 32 rows
    a.heads_per_wg = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    a.rows_per_wg = 32 * 8 / a.heads_per_wg;
  } else {
    // 4 waves of 32 rows of one head
    a.heads_per_wg = 1;
    a.rows_per_wg = 128;
  }
  a.nseg_q = nseg_q;
  const int64_t tps = (seg_len + a.rows_per_wg - 1) / a.rows_per_wg;
  const int64_t streams = (int64_t)a.batch * a.hkv;
  const int64_t total = streams * (G / a.heads_per_wg) * q_count * nseg_q * tps * a.kv_splits;
  if (tps > I32_MAX || total > I32_MAX) return fail(RA_ERR_INVALID_ARG, "problem too large for one launch");
  a.tiles_per_seg = (int32_t)tps;
  a.n_work = (int32_t)total;
  a.xcd_swizzle = (streams % 8 == 0) ? 1 : 0;
  // Ring mode walks every KV chunk of a stream.  When the K / V of all streams
  // would overflow the memory-side cache (256 MB; half of it is the budget
  // here) and exactly two streams fit, the streams run two at a time over all
  // XCDs (measured on the striped 128K workload, 8 streams of 64 MiB: 10.7 %
  // faster than one stream per XCD, results bitwise identical).  Smaller
  // streams keep one stream per XCD, whose L2 then serves their reuse.
  if (a.mode == ra::MODE_RING && streams % 8 == 0) {
    const int64_t kv_stream = 2 * a.seq * a.d * (bf16 ? 2 : 4);
    const int64_t budget = (int64_t)128 << 20;
    if (streams * kv_stream > budget && 2 * kv_stream <= budget && 4 * kv_stream > budget) a.xcd_swizzle = 2;
  }
  // Streams that do not split over the XCDs (one KV head, say): each XCD takes
  // blocks of 32 neighbouring workgroups, which walk the same keys in step.
  if (streams % 8 != 0 && total % 256 == 0) a.xcd_swizzle = 3;
  return RA_OK;
}

// The bf16 kernel addresses one head's K and V rows through buffer resources
// with 32-bit byte offsets, and keeps the table of the KV segments it walks in
// LDS (at most 1024 entries).
ra_status check_kv_span(const ra_attn_desc* d, int64_t kv_rows, int64_t runs) {
  if (d->in_dtype != RA_BF16) return RA_OK;
  const int64_t stride = (d->k.s > d->v.s ? d->k.s : d->v.s) * 2;
  if ((kv_rows - 1) * stride + d->d * 2 > I32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "one head's K or V rows span more than 2 GiB (rows x row stride)");
  if (runs > ra::BF16_MAX_RUNS)
    return fail(RA_ERR_UNSUPPORTED, "more than %d KV segments per call", (int)ra::BF16_MAX_RUNS);
  return RA_OK;
}

ra_status check_ring(const ra_ring_desc* r) {
  if (r == nullptr) return fail(RA_ERR_INVALID_ARG, "ring descriptor is NULL");
  if (r->kv_splits < 0 || r->kv_splits > RA_MAX_KV_SPLITS)
    return fail(RA_ERR_INVALID_ARG, "kv_splits must be in [0, %d]", RA_MAX_KV_SPLITS);
  if (r->n_chunks < 1 || r->seq < 1) return fail(RA_ERR_INVALID_ARG, "seq and n_chunks must be >= 1");
  if (r->seq % r->n_chunks) return fail(RA_ERR_INVALID_ARG, "seq (%lld) is not a multiple of n_chunks (%d)",
                                        (long long)r->seq, r->n_chunks);
  if (r->layout != RA_LAYOUT_CONTIGUOUS && r->layout != RA_LAYOUT_STRIPED && r->layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", r->layout);
  const int64_t L = r->seq / r->n_chunks;
  if (r->layout == RA_LAYOUT_ZIGZAG && (L % 2)) return fail(RA_ERR_INVALID_ARG, "zig-zag needs an even chunk length");
  if (r->causal != 0 && r->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (r->q_chunk_first < 0 || r->q_chunk_count < 1 || (int64_t)r->q_chunk_first + r->q_chunk_count > r->n_chunks)
    return fail(RA_ERR_INVALID_ARG, "query chunk range out of [0, n_chunks)");
  if (r->attn.lq != L || r->attn.lk != L)
    return fail(RA_ERR_INVALID_ARG, "attn.lq and attn.lk must equal seq / n_chunks (%lld)", (long long)L);
  if (r->seq > I32_MAX) return fail(RA_ERR_INVALID_ARG, "seq exceeds 2^31-1");
  return RA_OK;
}

// Descriptor checks of the backward (before any pointer is looked at).
ra_status check_bwd_desc(const ra_ring_desc* desc) {
  ra_status st = check_ring(desc);
  if (st != RA_OK) return st;
  if ((st = check_attn(&desc->attn)) != RA_OK) return st;
  const ra_attn_desc* d = &desc->attn;
  if (d->in_dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "the backward needs bf16 inputs (d = 128)");
  // dout is bf16 and read with the strides of out, in 16-byte pieces
  if (d->out.b % 8 || d->out.h % 8 || d->out.s % 8)
    return fail(RA_ERR_INVALID_ARG, "out strides must be multiples of 8 elements (dout is bf16 and shares them)");
  return RA_OK;
}

// Validation and planning of the backward, everything but the workspace:
// fills `a` (a.w left null) or returns the first rejection.
ra_status plan_bwd(const ra_ring_desc* desc, const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, float* dq, float* dk, float* dv, ra::BwdArgs& a) {
  ra_status st = check_bwd_desc(desc);
  if (st != RA_OK) return st;
  const ra_attn_desc* d = &desc->attn;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(RA_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk and dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(RA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t need = ra_ring_bwd_workspace_bytes(desc);
  if (need > (size_t)I32_MAX) return fail(RA_ERR_UNSUPPORTED, "more than 2^28 query rows x heads per call");
  const int64_t L = desc->seq / desc->n_chunks;
  const int64_t q_rows = (int64_t)desc->q_chunk_count * L;
  // query rows and dout rows of one head are addressed with 32-bit byte offsets
  const int64_t qstride = (d->q.s > d->out.s ? d->q.s : d->out.s) * 2;
  if ((q_rows - 1) * qstride + d->d * 2 > I32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "one head's query or dout rows span more than 2 GiB (rows x row stride)");
  const int32_t nseg = ra::num_segments(desc->layout);
  if ((st = check_kv_span(d, desc->seq, (int64_t)desc->n_chunks * nseg)) != RA_OK) return st;

  std::memset(&a, 0, sizeof(a));
  fill_common(a.f, d, q, k, v);
  a.f.out = const_cast<void*>(out);
  a.f.mode = ra::MODE_RING;
  a.f.causal = desc->causal;
  a.f.layout = desc->layout;
  a.f.n_chunks = desc->n_chunks;
  a.f.seq = desc->seq;
  a.f.q_first = desc->q_chunk_first;
  a.f.q_count = desc->q_chunk_count;
  a.f.lq = (int32_t)L;
  a.f.lk = (int32_t)L;
  if ((st = plan_launch(a.f, true, L / nseg, nseg, desc->q_chunk_count)) != RA_OK) return st;
  a.dout = dout;
  a.lse_in = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.w = nullptr;
  a.q_rows = (int32_t)q_rows;
  a.scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->d));
  const int64_t kv_tps = (L / nseg + 255) / 256;
  const int64_t n_kv = (int64_t)d->batch * d->hkv * desc->n_chunks * nseg * kv_tps;
  if (n_kv > I32_MAX) return fail(RA_ERR_INVALID_ARG, "problem too large for one launch");
  a.kv_tiles_per_seg = (int32_t)kv_tps;
  a.n_work_kv = (int32_t)n_kv;
  return RA_OK;
}

// The three backward launches, in order, on one stream.
ra_status launch_bwd(const ra::BwdArgs& a, hipStream_t s0, const char* who) {
  char what[96];
  ra_status st;
  std::snprintf(what, sizeof(what), "%s (prep)", who);
  if ((st = hip_status(ra::launch_bwd_prep(a, s0), what)) != RA_OK) return st;
  std::snprintf(what, sizeof(what), "%s (dq)", who);
  if ((st = hip_status(ra::launch_attn_bwd_dq_bf16(a, s0), what)) != RA_OK) return st;
  std::snprintf(what, sizeof(what), "%s (dk, dv)", who);
  return hip_status(ra::launch_attn_bwd_dkdv_bf16(a, s0), what);
}

}  // namespace

extern "C" {

int ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_INVALID_ARG: return "invalid argument";
    case RA_ERR_UNSUPPORTED: return "unsupported";
    case RA_ERR_WORKSPACE: return "workspace too small";
    case RA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ra_last_error(void) { return g_err; }

ra_status ra_state_init(const ra_attn_desc* desc, float* m, float* l, float* o, ra_stream stream) {
  ra_status st = check_attn(desc);
  if (st != RA_OK) return st;
  if (!m || !l || !o) return fail(RA_ERR_INVALID_ARG, "m, l and o must be non-NULL");
  if (!aligned16(o)) return fail(RA_ERR_INVALID_ARG, "o must be 16-byte aligned");
  return hip_status(ra::launch_state_init(rows_args(desc), m, l, o, (hipStream_t)stream), "ra_state_init");
}

ra_status ra_chunk_fwd(const ra_attn_desc* desc, const void* q, const void* k, const void* v, float* m, float* l,
                       float* o, int64_t causal_delta, int32_t causal, ra_stream stream) {
  ra_status st = check_attn(desc);
  if (st != RA_OK) return st;
  if (!q || !k || !v || !m || !l || !o) return fail(RA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(RA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (causal != 0 && causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  ra::FwdArgs a;
  fill_common(a, desc, q, k, v);
  a.m = m; a.l = l; a.o = o;
  a.mode = ra::MODE_CHUNK;
  a.causal = causal;
  a.lq = (int32_t)desc->lq;
  a.lk = (int32_t)desc->lk;
  a.delta = causal ? causal_delta : 0;
  a.n_chunks = 1;
  a.q_count = 1;
  const bool bf16 = desc->in_dtype == RA_BF16;
  if ((st = check_kv_span(desc, desc->lk, 1)) != RA_OK) return st;
  if ((st = plan_launch(a, bf16, desc->lq, 1, 1)) != RA_OK) return st;
  // a causal offset below -(lq - 1) hides every key: nothing to do
  if (causal && causal_delta < -(desc->lq - 1)) return RA_OK;
  return hip_status(bf16 ? ra::launch_attn_fwd_bf16(a, (hipStream_t)stream)
                         : ra::launch_attn_fwd_f32(a, (hipStream_t)stream),
                    "ra_chunk_fwd");
}

ra_status ra_finalize(const ra_attn_desc* desc, const float* m, const float* l, const float* o, void* out,
                      float* lse, ra_stream stream) {
  ra_status st = check_attn(desc);
  if (st != RA_OK) return st;
  if (!m || !l || !o || !out) return fail(RA_ERR_INVALID_ARG, "m, l, o and out must be non-NULL");
  if (!aligned16(o) || !aligned16(out)) return fail(RA_ERR_INVALID_ARG, "o and out must be 16-byte aligned");
  return hip_status(ra::launch_finalize(rows_args(desc), m, l, o, out, desc->out_dtype == RA_BF16, lse,
                                        (hipStream_t)stream),
                    "ra_finalize");
}

ra_status ra_merge(const ra_attn_desc* desc, const float* lse_a, const float* o_a, const float* lse_b,
                   const float* o_b, float* lse_out, float* o_out, ra_stream stream) {
  ra_status st = check_attn(desc);
  if (st != RA_OK) return st;
  if (!lse_a || !o_a || !lse_b || !o_b || !lse_out || !o_out)
    return fail(RA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out))
    return fail(RA_ERR_INVALID_ARG, "o tensors must be 16-byte aligned");
  return hip_status(ra::launch_merge(rows_args(desc), lse_a, o_a, lse_b, o_b, lse_out, o_out, (hipStream_t)stream),
                    "ra_merge");
}

size_t ra_ring_workspace_bytes(const ra_ring_desc* desc) {
  if (desc == nullptr || desc->n_chunks < 1 || desc->kv_splits <= 1) return 0;
  const int64_t rows = (int64_t)desc->q_chunk_count * (desc->seq / desc->n_chunks);
  return (size_t)((int64_t)desc->kv_splits * desc->attn.batch * desc->attn.hq * rows * (desc->attn.d + 1) *
                  (int64_t)sizeof(float));
}

ra_status ra_ring_fwd(const ra_ring_desc* desc, const void* q, const void* k, const void* v, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, ra_stream stream) {
  ra_status st = check_ring(desc);
  if (st != RA_OK) return st;
  if ((st = check_attn(&desc->attn)) != RA_OK) return st;
  if (!q || !k || !v || !out) return fail(RA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(RA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  const size_t ws_need = ra_ring_workspace_bytes(desc);
  if (workspace_bytes < ws_need) return fail(RA_ERR_WORKSPACE, "workspace too small (%zu bytes needed)", ws_need);
  if (ws_need > 0 && (workspace == nullptr || !aligned16(workspace)))
    return fail(RA_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned when kv_splits > 1");
  const ra_attn_desc* d = &desc->attn;
  ra::FwdArgs a;
  fill_common(a, d, q, k, v);
  a.out = out;
  a.lse = lse;
  a.mode = ra::MODE_RING;
  a.causal = desc->causal;
  a.layout = desc->layout;
  a.n_chunks = desc->n_chunks;
  a.seq = desc->seq;
  a.q_first = desc->q_chunk_first;
  a.q_count = desc->q_chunk_count;
  a.lq = (int32_t)d->lq;
  a.lk = (int32_t)d->lk;
  const int32_t nseg = ra::num_segments(desc->layout);
  const bool bf16 = d->in_dtype == RA_BF16;
  if ((st = check_kv_span(d, desc->seq, (int64_t)desc->n_chunks * nseg)) != RA_OK) return st;
  const int32_t S = desc->kv_splits > 1 ? desc->kv_splits : 1;
  const int64_t rows = (int64_t)desc->q_chunk_count * d->lq;
  a.kv_splits = S;
  if (S > 1) {
    if (rows > I32_MAX) return fail(RA_ERR_INVALID_ARG, "query rows exceed 2^31-1");
    a.part_rows = (int32_t)rows;
    a.part_o = (float*)workspace;
    a.part_lse = (float*)workspace + (int64_t)S * d->batch * d->hq * rows * d->d;
  }
  if ((st = plan_launch(a, bf16, d->lq / nseg, nseg, desc->q_chunk_count)) != RA_OK) return st;
  st = hip_status(bf16 ? ra::launch_attn_fwd_bf16(a, (hipStream_t)stream)
                       : ra::launch_attn_fwd_f32(a, (hipStream_t)stream),
                  "ra_ring_fwd");
  if (st != RA_OK || S == 1) return st;
  ra::RowsArgs g;
  g.batch = (int32_t)d->batch;
  g.heads = (int32_t)d->hq;
  g.rows = (int32_t)rows;
  g.d = (int32_t)d->d;
  g.ml_sb = d->ml.b; g.ml_sh = d->ml.h;
  g.o_sb = g.o_sh = g.o_ss = 0;
  g.out_sb = d->out.b; g.out_sh = d->out.h; g.out_ss = d->out.s;
  return hip_status(ra::launch_split_merge(g, S, a.part_lse, a.part_o, out, a.out_bf16, lse, (hipStream_t)stream),
                    "ra_ring_fwd (split merge)");
}

ra_status ra_ring_step(const ra_ring_desc* desc, int32_t step, const void* q, const void* k, const void* v, float* m,
                       float* l, float* o, ra_stream stream) {
  ra_status st = check_ring(desc);
  if (st != RA_OK) return st;
  if ((st = check_attn(&desc->attn)) != RA_OK) return st;
  if (desc->q_chunk_count != 1) return fail(RA_ERR_INVALID_ARG, "ra_ring_step takes one query chunk (q_chunk_count = 1)");
  if (step < 0 || step >= desc->n_chunks) return fail(RA_ERR_INVALID_ARG, "step %d out of [0, n_chunks)", step);
  if (!q || !k || !v || !m || !l || !o) return fail(RA_ERR_INVALID_ARG, "q, k, v, m, l and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(RA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  const ra_attn_desc* d = &desc->attn;
  const int32_t nseg = ra::num_segments(desc->layout);
  const int32_t qc = desc->q_chunk_first;
  const int32_t j = ra::ring_kv_chunk(qc, step, desc->n_chunks);
  // Query segments with a visible key in this step.  Nothing to do when there
  // is none; in the zig-zag layout the late segment always sees the step's
  // chunk and the early one only when that chunk is not later than its own,
  // so otherwise only the late segment's workgroups are launched (the work
  // decomposition puts the late segment first).
  bool seg_live[2] = {true, true};
  if (desc->causal) {
    for (int qs = 0; qs < nseg; ++qs) {
      seg_live[qs] = false;
      const ra::Segment a = ra::segment(desc->layout, desc->seq, desc->n_chunks, qc, qs);
      for (int ks = 0; ks < nseg; ++ks) {
        const ra::Segment b = ra::segment(desc->layout, desc->seq, desc->n_chunks, j, ks);
        if (ra::pair_kind(ra::pair_delta(a, b), a.len, b.len) != RA_SKIP) seg_live[qs] = true;
      }
    }
    if (!seg_live[0] && (nseg == 1 || !seg_live[1])) return RA_OK;
  }
  const int32_t nseg_launch = (nseg == 2 && !seg_live[0]) ? 1 : nseg;
  const bool bf16 = d->in_dtype == RA_BF16;
  if ((st = check_kv_span(d, d->lk, nseg)) != RA_OK) return st;
  ra::FwdArgs a;
  fill_common(a, d, q, k, v);
  a.m = m; a.l = l; a.o = o;
  a.mode = ra::MODE_STEP;
  a.causal = desc->causal;
  a.layout = desc->layout;
  a.n_chunks = desc->n_chunks;
  a.seq = desc->seq;
  a.q_first = qc;
  a.q_count = 1;
  a.step = step;
  a.lq = (int32_t)d->lq;
  a.lk = (int32_t)d->lk;
  if ((st = plan_launch(a, bf16, d->lq / nseg, nseg_launch, 1)) != RA_OK) return st;
  return hip_status(bf16 ? ra::launch_attn_fwd_bf16(a, (hipStream_t)stream)
                         : ra::launch_attn_fwd_f32(a, (hipStream_t)stream),
                    "ra_ring_step");
}

ra_status ra_ring_kv_splits_hint(const ra_ring_desc* desc, int32_t* splits) {
  ra_status st = check_ring(desc);
  if (st != RA_OK) return st;
  if ((st = check_attn(&desc->attn)) != RA_OK) return st;
  if (splits == nullptr) return fail(RA_ERR_INVALID_ARG, "splits is NULL");
  const ra_attn_desc* d = &desc->attn;
  const bool bf16 = d->in_dtype == RA_BF16;
  ra::FwdArgs a;
  fill_common(a, d, nullptr, nullptr, nullptr);
  const int32_t nseg = ra::num_segments(desc->layout);
  if ((st = plan_launch(a, bf16, d->lq / nseg, nseg, desc->q_chunk_count)) != RA_OK) return st;
  // Below two workgroups per compute unit (a bf16 workgroup fills one, an
  // fp32 one of 4 waves about half of one), split to about four, so that short
  // ranges also even out query tiles of different causal work; never more
  // ranges than about one per four KV tiles of 64 keys of the sequence.
  const int64_t enough = bf16 ? 512 : 1024;
  int64_t s = a.n_work >= enough ? 1 : (2 * enough + a.n_work - 1) / a.n_work;
  const int64_t cap = desc->seq / 256 > 1 ? desc->seq / 256 : 1;
  if (s > cap) s = cap;
  if (s > RA_MAX_KV_SPLITS) s = RA_MAX_KV_SPLITS;
  *splits = (int32_t)(s < 1 ? 1 : s);
  return RA_OK;
}

size_t ra_ring_bwd_workspace_bytes(const ra_ring_desc* desc) {
  if (desc == nullptr || desc->n_chunks < 1) return 0;
  const int64_t rows = (int64_t)desc->q_chunk_count * (desc->seq / desc->n_chunks);
  return (size_t)(2 * desc->attn.batch * desc->attn.hq * rows * (int64_t)sizeof(float));
}

ra_status ra_ring_bwd(const ra_ring_desc* desc, const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, float* dq, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, ra_stream stream) {
  ra::BwdArgs a;
  ra_status st = plan_bwd(desc, q, k, v, out, dout, lse, dq, dk, dv, a);
  if (st != RA_OK) return st;
  if (workspace == nullptr || !aligned16(workspace))
    return fail(RA_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");
  const size_t need = ra_ring_bwd_workspace_bytes(desc);
  if (workspace_bytes < need) return fail(RA_ERR_WORKSPACE, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
  a.w = static_cast<float*>(workspace);
  return launch_bwd(a, (hipStream_t)stream, "ra_ring_bwd");
}

ra_status ra_ring_bwd_noalloc(const ra_ring_desc* desc, const void* q, const void* k, const void* v,
                              const void* out, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                              ra_stream stream) {
  ra::BwdArgs a;
  ra_status st = plan_bwd(desc, q, k, v, out, dout, lse, dq, dk, dv, a);
  if (st != RA_OK) return st;
  const size_t need = ra_ring_bwd_workspace_bytes(desc);
  static_assert(ra::BWD_SCRATCH_BYTES == RA_BWD_NOALLOC_MAX_BYTES, "scratch size and header limit differ");
  if (need > (size_t)RA_BWD_NOALLOC_MAX_BYTES)
    return fail(RA_ERR_UNSUPPORTED, "ra_ring_bwd_noalloc: the call needs %zu workspace bytes, more than its %u "
                "(at most %u batch x query heads x query rows); use ra_ring_bwd with a workspace",
                need, (unsigned)RA_BWD_NOALLOC_MAX_BYTES, (unsigned)(RA_BWD_NOALLOC_MAX_BYTES / 8));
  void* ws = nullptr;
  if ((st = hip_status(ra::bwd_scratch((hipStream_t)stream, &ws), "ra_ring_bwd_noalloc (scratch lookup)")) != RA_OK)
    return st;
  a.w = static_cast<float*>(ws);
  return launch_bwd(a, (hipStream_t)stream, "ra_ring_bwd_noalloc");
}

ra_status ra_layout_positions(int32_t layout, int64_t seq, int32_t n_chunks, int32_t chunk, int64_t* pos) {
  if (pos == nullptr) return fail(RA_ERR_INVALID_ARG, "pos is NULL");
  if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED && layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
  if (n_chunks < 1 || seq < 1 || seq % n_chunks) return fail(RA_ERR_INVALID_ARG, "seq must be a multiple of n_chunks");
  const int64_t L = seq / n_chunks;
  if (layout == RA_LAYOUT_ZIGZAG && (L % 2)) return fail(RA_ERR_INVALID_ARG, "zig-zag needs an even chunk length");
  if (chunk < 0 || chunk >= n_chunks) return fail(RA_ERR_INVALID_ARG, "chunk out of range");
  for (int64_t p = 0; p < L; ++p) pos[p] = ra::position(layout, seq, n_chunks, chunk, p);
  return RA_OK;
}

ra_status ra_ring_schedule(const ra_ring_desc* desc, int32_t q_chunk, ra_task* tasks, int32_t capacity,
                           int32_t* n_tasks) {
  ra_status st = check_ring(desc);
  if (st != RA_OK) return st;
  if (n_tasks == nullptr) return fail(RA_ERR_INVALID_ARG, "n_tasks is NULL");
  if (q_chunk < 0 || q_chunk >= desc->n_chunks) return fail(RA_ERR_INVALID_ARG, "q_chunk out of range");
  const int32_t n = desc->n_chunks;
  const int32_t nseg = ra::num_segments(desc->layout);
  const int64_t count = (int64_t)n * nseg * nseg;
  if (count > I32_MAX) return fail(RA_ERR_INVALID_ARG, "schedule too long");
  *n_tasks = (int32_t)count;
  if (capacity < count || (count > 0 && tasks == nullptr))
    return fail(RA_ERR_INVALID_ARG, "capacity %d < %lld tasks", capacity, (long long)count);
  int32_t idx = 0;
  for (int32_t t = 0; t < n; ++t) {
    const int32_t j = ra::ring_kv_chunk(q_chunk, t, n);
    for (int qs = 0; qs < nseg; ++qs) {
      const ra::Segment qseg = ra::segment(desc->layout, desc->seq, n, q_chunk, qs);
      for (int ks = 0; ks < nseg; ++ks) {
        const ra::Segment kseg = ra::segment(desc->layout, desc->seq, n, j, ks);
        ra_task& e = tasks[idx++];
        e.step = t;
        e.kv_chunk = j;
        e.q_row0 = qseg.row0;
        e.q_len = qseg.len;
        e.kv_row0 = kseg.row0;
        e.kv_len = kseg.len;
        e.reserved = 0;
        if (desc->causal) {
          e.delta = ra::pair_delta(qseg, kseg);
          e.kind = ra::pair_kind(e.delta, qseg.len, kseg.len);
        } else {
          e.delta = 0;
          e.kind = RA_FULL;
        }
      }
    }
  }
  return RA_OK;
}

ra_status ra_permute_strided(int32_t layout, int32_t to_chunked, int64_t batch, int64_t heads, int64_t seq,
                             int32_t n_chunks, int64_t d, int32_t dtype, const void* src, int64_t src_sb,
                             int64_t src_sh, int64_t src_ss, void* dst, int64_t dst_sb, int64_t dst_sh,
                             int64_t dst_ss, ra_stream stream) {
  if (!src || !dst) return fail(RA_ERR_INVALID_ARG, "src and dst must be non-NULL");
  if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED && layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || heads < 1 || d < 1 || n_chunks < 1 || seq < 1 || seq % n_chunks)
    return fail(RA_ERR_INVALID_ARG, "bad shape");
  if (layout == RA_LAYOUT_ZIGZAG && ((seq / n_chunks) % 2))
    return fail(RA_ERR_INVALID_ARG, "zig-zag needs an even chunk length");
  if (to_chunked != 0 && to_chunked != 1) return fail(RA_ERR_INVALID_ARG, "to_chunked must be 0 or 1");
  const int64_t strides[6] = {src_sb, src_sh, src_ss, dst_sb, dst_sh, dst_ss};
  for (int64_t st : strides)
    if (st < 0) return fail(RA_ERR_INVALID_ARG, "strides must not be negative");
  const int64_t eb = elem_bytes(dtype);
  const int64_t row_bytes = d * eb;
  // every piece a thread moves must be a whole number of elements inside one row: the widest of 16,
  // 8, 4, 2 bytes that divides the row, both pointers and every stride in bytes
  uint64_t bits = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | (uint64_t)row_bytes;
  for (int64_t st : strides) bits |= (uint64_t)(st * eb);
  if (bits % eb) return fail(RA_ERR_INVALID_ARG, "misaligned pointer");
  int unit = 16;
  while (bits % unit) unit >>= 1;
  ra::PermuteArgs p;
  p.layout = layout;
  p.to_chunked = to_chunked;
  p.n_chunks = n_chunks;
  p.batch = batch;
  p.heads = heads;
  p.seq = seq;
  p.units_per_row = row_bytes / unit;
  p.src_sb = src_sb * eb / unit;
  p.src_sh = src_sh * eb / unit;
  p.src_ss = src_ss * eb / unit;
  p.dst_sb = dst_sb * eb / unit;
  p.dst_sh = dst_sh * eb / unit;
  p.dst_ss = dst_ss * eb / unit;
  return hip_status(ra::launch_permute(p, unit, src, dst, (hipStream_t)stream), "ra_permute");
}

ra_status ra_permute(int32_t layout, int32_t to_chunked, int64_t batch, int64_t heads, int64_t seq,
                     int32_t n_chunks, int64_t d, int32_t dtype, const void* src, void* dst, ra_stream stream) {
  // contiguous [batch, heads, seq, d]; the strides overflow only for shapes no buffer can hold
  if (batch < 1 || heads < 1 || d < 1 || seq < 1) return fail(RA_ERR_INVALID_ARG, "bad shape");
  return ra_permute_strided(layout, to_chunked, batch, heads, seq, n_chunks, d, dtype, src, heads * seq * d,
                            seq * d, d, dst, heads * seq * d, seq * d, d, stream);
}

}  // extern "C"
