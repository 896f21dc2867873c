// Internal interface between the C ABI (ringattn_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Arguments of the fused attention-forward kernels.  One launch covers a
// single chunk update with the running state in HBM (mode CHUNK), the whole
// ring for a range of query chunks with the state kept on chip and the output
// finalized at the end (mode RING), or one ring step of one query chunk with
// that step's KV chunk in its own buffer and the running state in HBM (mode
// STEP: what each device of a ring runs when a KV chunk arrives).
enum FwdMode : int32_t { MODE_CHUNK = 0, MODE_RING = 1, MODE_STEP = 2 };

// The bf16 kernel keeps the table of the KV segments one workgroup walks in
// LDS; a call may cover at most this many (ring steps x segments per chunk).
constexpr int32_t BF16_MAX_RUNS = 1024;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  // running state (MODE_CHUNK, MODE_STEP): m, l [B, Hq, Lq]; o [B, Hq, Lq, d]
  float* m;
  float* l;
  float* o;
  int64_t ml_sb, ml_sh;
  int64_t o_sb, o_sh, o_ss;
  // normalized output and lse (MODE_RING); lse may be null
  void* out;
  int64_t out_sb, out_sh, out_ss;
  float* lse;
  int32_t out_bf16;
  int32_t batch, hq, hkv, d;
  int32_t mode;
  int32_t causal;
  // ring geometry (MODE_RING, MODE_STEP): chunk length L, layout, N chunks;
  // MODE_STEP computes ring step `step` of query chunk q_first (q_count = 1)
  // and its K / V rows are those of KV chunk (q_first - step) mod N only
  int32_t layout;
  int32_t n_chunks;
  int64_t seq;
  int32_t q_first, q_count;
  int32_t step;
  // chunk geometry (MODE_CHUNK): lq query rows, lk key rows, one offset
  int32_t lq, lk;
  int64_t delta;
  float scale_log2;  // scale * log2(e)
  // work decomposition, filled by the host planner
  int32_t heads_per_wg;   // query heads of one KV head handled by one workgroup
  int32_t rows_per_wg;    // query rows of one segment handled by one workgroup
  int32_t nseg_q;         // query segments per query chunk (2 for zig-zag)
  int32_t tiles_per_seg;  // workgroups along one query segment
  int32_t xcd_swizzle;    // 1: one KV stream per XCD; 2 or 4: streams that many at a time over all XCDs;
                          // 3: blocks of 32 workgroups, block b on XCD b % 8
  int32_t n_work;         // total workgroups
  // split-KV (MODE_RING): each query tile's KV tiles, in ring order, are cut
  // into kv_splits consecutive ranges of (nearly) equal tile counts, one
  // workgroup each; every range writes its normalized partial o and its
  // natural lse (lse = -inf, o = 0 for an empty range) to part_o / part_lse,
  // [kv_splits][B][Hq][part_rows](+[d]) fp32, row index = query buffer row.
  int32_t kv_splits;      // 1: no split, the kernel finalizes out / lse itself
  int32_t part_rows;
  float* part_o;
  float* part_lse;
};

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream);

// Arguments of the backward kernels (bf16 inputs, d = 128, ring mode).  `f`
// carries q, k, v, their strides, the ring geometry and the dQ work
// decomposition (the forward's); out and dout share the out strides.
struct BwdArgs {
  FwdArgs f;
  const void* dout;
  const float* lse_in;  // natural log-sum-exp of the forward, strides f.ml_sb / f.ml_sh
  float* dq;            // fp32, strides of q
  float* dk;            // fp32, strides of k
  float* dv;            // fp32, strides of v
  float* w;             // workspace: two fp32 per (b, query head, row), see launch_bwd_prep
  int32_t q_rows;       // query rows per (b, head): q_count * L
  float scale;          // score scale
  // dK/dV work decomposition: key tiles of 256 rows per KV segment
  int32_t kv_tiles_per_seg;
  int32_t n_work_kv;
};

// w[0 .. B*Hq*q_rows): -lse / scale (a large negative value for lse = -inf);
// w[B*Hq*q_rows ..): -rowsum(dout * out)
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream);

// The backward's workspace without an allocation: the device address, on the
// GPU that `stream` belongs to (the current GPU for the null stream), of a
// file-scope array of BWD_SCRATCH_BYTES bytes (256-byte aligned).  Looked up
// once per GPU; every call on that GPU shares the array.
constexpr size_t BWD_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t bwd_scratch(hipStream_t stream, void** ptr);

struct RowsArgs {  // [B, H, rows] fp32 tensors with strides (b, h), row stride 1; o-like with (b, h, s)
  int32_t batch, heads, rows, d;
  int64_t ml_sb, ml_sh;
  int64_t o_sb, o_sh, o_ss;
  int64_t out_sb, out_sh, out_ss;
};

hipError_t launch_state_init(const RowsArgs& g, float* m, float* l, float* o, hipStream_t stream);
hipError_t launch_finalize(const RowsArgs& g, const float* m, const float* l, const float* o, void* out,
                           int32_t out_bf16, float* lse, hipStream_t stream);
hipError_t launch_merge(const RowsArgs& g, const float* lse_a, const float* o_a, const float* lse_b,
                        const float* o_b, float* lse_out, float* o_out, hipStream_t stream);
// out / lse of the rows of [B, H, rows] from kv_splits partials (the layout of
// FwdArgs::part_o / part_lse): lse = M + ln sum_s e^(lse_s - M), M = max_s lse_s,
// out = sum_s e^(lse_s - lse) o_s; a row with every lse_s = -inf gets out = 0,
// lse = -inf.  g gives the out / lse strides (ml_*, out_*); lse may be null.
hipError_t launch_split_merge(const RowsArgs& g, int32_t kv_splits, const float* part_lse, const float* part_o,
                              void* out, int32_t out_bf16, float* lse, hipStream_t stream);
// Row permutation between logical and chunk-major order.  Strides are in
// `unit`-byte pieces ([batch, head, row] of src, then of dst); a row is
// row_bytes / unit pieces, contiguous.
struct PermuteArgs {
  int32_t layout, to_chunked, n_chunks;
  int64_t batch, heads, seq, units_per_row;
  int64_t src_sb, src_sh, src_ss, dst_sb, dst_sh, dst_ss;
};
hipError_t launch_permute(const PermuteArgs& p, int unit, const void* src, void* dst, hipStream_t stream);

}  // namespace ra
