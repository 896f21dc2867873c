// Ring-ordered exact attention forward, fp32 inputs (d in {16, 32, 64, 128}).
//
// The fp32 path serves small, precision-sensitive cases (the four-device
// simulation of the glossary page is fp32 with d = 16); gfx950 has no
// reduced-precision fp32 matrix mode, so a per-row VALU kernel keeps the
// arithmetic in true fp32.  One wave per workgroup, one query row per lane,
// K / V tiles of 64 keys staged through LDS.  Same schedule, same masking
// rule and same (m, l, o) update as the bf16 kernel: per tile, the new row
// maximum, the rescale factor 2^(m - m'), then the tile's exponentials.
#include <hip/hip_runtime.h>

#include "fwd_common.h"
#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

constexpr int BN = 64;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

template <int D>
__global__ __launch_bounds__(64, 1) void attn_fwd_f32_kernel(FwdArgs a) {
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int lane = threadIdx.x;

  const WorkItem it = decode_work(a, blockIdx.x);
  const QGeom qg = query_geom(a, it);
  const int G = a.hq / a.hkv;
  const int h = it.kvh * G + it.hg;
  const int p0 = it.tile * a.rows_per_wg;
  const int p_hi = min(p0 + a.rows_per_wg, qg.len) - 1;
  const int p = p0 + lane;
  const bool row_ok = p < qg.len;

  const float* Qg = (const float*)a.q + (int64_t)it.b * a.q_sb + (int64_t)h * a.q_sh;
  const float* Kg = (const float*)a.k + (int64_t)it.b * a.k_sb + (int64_t)it.kvh * a.k_sh;
  const float* Vg = (const float*)a.v + (int64_t)it.b * a.v_sb + (int64_t)it.kvh * a.v_sh;

  float q[D], acc[D];
  float m_run = -INFINITY, l_run = 0.f;
  // chunk / step modes: the incoming m (natural) and its base-2 image; a row
  // whose maximum does not move hands m back unchanged, not re-rounded
  float m_in = -INFINITY, m_in2 = -INFINITY;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = row_ok ? Qg[(qg.row_base + p) * a.q_ss + e] : 0.f;
    acc[e] = 0.f;
  }
  if (a.mode != MODE_RING && row_ok) {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + p;
    m_in = a.m[mi];
    m_run = m_in2 = m_in == -INFINITY ? -INFINITY : m_in * LOG2E;
    l_run = a.l[mi];
    const float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + p) * a.o_ss;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = orow[e];
  }
  const float c2 = a.scale_log2;

  TileCursor<BN> cur = make_cursor<BN>(a, qg, p_hi);
  int64_t left = INT64_MAX;
  if (a.kv_splits > 1) {
    // this workgroup's range of the walk: tiles [T s / S, T (s + 1) / S)
    TileCursor<BN> c = cur;
    int64_t total = 0;
    for (; !c.done; c.advance()) ++total;
    const int64_t tb = total * it.split / a.kv_splits, te = total * (it.split + 1) / a.kv_splits;
    for (int64_t i = 0; i < tb; ++i) cur.advance();
    left = te - tb;
  }
  for (; !cur.done && left > 0; --left) {
    __syncthreads();
    for (int i = lane; i < BN * D; i += 64) {
      const int r = i / D, e = i - r * D;
      const bool ok = cur.k0 + r < cur.kv_len;
      const int64_t row = cur.kv_row + cur.k0 + r;
      ks[r][e] = ok ? Kg[row * a.k_ss + e] : 0.f;
      vs[r][e] = ok ? Vg[row * a.v_ss + e] : 0.f;
    }
    __syncthreads();
    int64_t lim = (int64_t)cur.kv_len - 1 - cur.k0;
    if (a.causal) {
      const int64_t lc = (int64_t)p + cur.delta - cur.k0;
      lim = lc < lim ? lc : lim;
    }
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) d = fmaf(q[e], ks[j][e], d);
      s[j] = (j > lim) ? -INFINITY : d;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pv = exp2f(fmaf(s[j], c2, -m_use));
      l_run += pv;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pv, vs[j][e], acc[e]);
    }
    cur.advance();
  }

  if (!row_ok) return;
  if (a.mode == MODE_RING && a.kv_splits > 1) {
    // partial of this KV range: normalized o and natural lse
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t prow = (((int64_t)it.split * a.batch + it.b) * a.hq + h) * a.part_rows + qg.row_base + p;
#pragma unroll
    for (int e = 0; e < D; ++e) a.part_o[prow * D + e] = acc[e] * inv;
    a.part_lse[prow] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
  } else if (a.mode == MODE_RING) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t orow = (int64_t)it.b * a.out_sb + (int64_t)h * a.out_sh + (qg.row_base + p) * a.out_ss;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      if (a.out_bf16) ((__bf16*)a.out)[orow + e] = (__bf16)(acc[e] * inv);
      else ((float*)a.out)[orow + e] = acc[e] * inv;
    }
    if (a.lse != nullptr) {
      const int64_t li = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + p;
      a.lse[li] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
    }
  } else {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + p;
    a.m[mi] = m_run == m_in2 ? m_in : m_run * LN2;
    a.l[mi] = l_run;
    float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + p) * a.o_ss;
#pragma unroll
    for (int e = 0; e < D; ++e) orow[e] = acc[e];
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
  switch (a.d) {
    case 16: hipLaunchKernelGGL(attn_fwd_f32_kernel<16>, dim3(a.n_work), dim3(64), 0, stream, a); break;
    case 32: hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, dim3(a.n_work), dim3(64), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(a.n_work), dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(a.n_work), dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
