// Ring-ordered exact attention forward, fp32 inputs (d in {16, 32, 64, 128}),
// on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: exact fp32 products,
// fp32 accumulation, so the arithmetic stays in true fp32).
//
// The fp32 path serves the small, precision-bound cases (the four-device
// simulation of the glossary page is fp32 with d = 16) and fp32 callers.  A
// workgroup is 4 waves of 32 query rows of one query head; K / V tiles of 32
// keys are staged through LDS and read by the 4 waves.  Per tile, with
// c = scale * log2(e), the pages' update in base 2:
//   S^T = K Q^T                        (d / 2 MFMA)
//   mask (keys past the segment end, pairs past the diagonal)
//   m'  = max(m, c * rowmax S),  a = 2^(m - m')
//   P   = 2^(c S - m'),  l = a l + rowsum P
//   O^T = a O^T + V^T P^T              (32 MFMA per 32 rows of O^T)
// S is computed transposed (32 keys x 32 queries): one query per lane, so the
// row maximum is in-lane plus one exchange with lane l ^ 32, and a lane's 16
// scores are exactly the P^T operands of its 16 PV products.
//
// Operand layouts (32x32x2 fp32: lane l gives A[l % 32][l / 32] and
// B[l / 32][l % 32]; the result holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32 in register r):
//   * QK product j = 4 m + e uses head dimension 8 m + 4 g + e in lane half
//     g = l / 32, so a lane's Q values (registers) and K values (one 16-byte LDS
//     read per four products) are contiguous float4 pieces;
//   * PV product j' pairs key 8 (j' / 4) + e with key 8 (j' / 4) + 4 + e
//     (e = j' % 4), the keys the two lane halves hold in register j' of S^T;
//     V is stored in LDS four keys to a float4 (V[4 q .. 4 q + 3][dv]), so one
//     16-byte read gives four products' A operands.
#include <hip/hip_runtime.h>

#include "fwd_common.h"
#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 32;            // keys per tile
constexpr int NWAVES = 4;         // 32 query rows each
constexpr int NTHREADS = 64 * NWAVES;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ f32x16 mfma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// max / sum of a value and the one held by lane l ^ 32
__device__ __forceinline__ float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(NTHREADS) void attn_fwd_f32_kernel(FwdArgs a) {
  constexpr int DP = D < 32 ? 32 : D;  // rows of O^T, a whole number of 32-row blocks
  constexpr int NDB = DP / 32;         // O^T blocks
  constexpr int NC = D / 4;            // float4 pieces of one row
  constexpr int NM = D / 8;            // QK read steps (four products each)
  // K tile: blocks of 16 rows, piece c of the 16 rows side by side (a 16-lane
  // read of one piece covers 256 contiguous bytes); V tile: V[4 q + i][dv] at
  // float4 q * DP + dv, component i (dv >= D stays zero)
  __shared__ f32x4 ks[BN * NC];
  __shared__ f32x4 vt[(BN / 4) * DP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const WorkItem it = decode_work(a, blockIdx.x);
  const QGeom qg = query_geom(a, it);
  const int G = a.hq / a.hkv;
  const int h = it.kvh * G + it.hg;
  const int wg_p0 = it.tile * a.rows_per_wg;
  const int wg_p_hi = min(wg_p0 + a.rows_per_wg, qg.len) - 1;
  const int my_p = wg_p0 + 32 * wave + l32;   // this lane's query row
  const bool row_ok = my_p < qg.len;

  const float* Qg = (const float*)a.q + (int64_t)it.b * a.q_sb + (int64_t)h * a.q_sh;
  const float* Kg = (const float*)a.k + (int64_t)it.b * a.k_sb + (int64_t)it.kvh * a.k_sh;
  const float* Vg = (const float*)a.v + (int64_t)it.b * a.v_sb + (int64_t)it.kvh * a.v_sh;

  // Q of this lane's row as B operands: qv[m] = Q[row][8 m + 4 g .. + 3]
  f32x4 qv[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
    qv[m] = row_ok ? *(const f32x4*)(Qg + (qg.row_base + my_p) * a.q_ss + 8 * m + 4 * g) : f32x4{};

  // running state (log2 units); l_run is this half-wave's partial sum
  float m_run = -INFINITY, l_run = 0.f;
  // chunk / step modes: the incoming m (natural) and its base-2 image; a row
  // whose maximum does not move hands m back unchanged, not re-rounded
  float m_in = -INFINITY, m_in2 = -INFINITY;
  f32x16 acc[NDB];  // acc[b]: O^T[dv = 32 b + 8 (r / 4) + 4 g + r % 4][query my_p]
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};
  if (a.mode != MODE_RING && row_ok) {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
    m_in = a.m[mi];
    m_run = m_in2 = m_in == -INFINITY ? -INFINITY : m_in * LOG2E;
    l_run = g == 0 ? a.l[mi] : 0.f;
    const float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + my_p) * a.o_ss;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv = 32 * b + 8 * r4 + 4 * g;
        if (dv < D) {
          const f32x4 v4 = *(const f32x4*)(orow + dv);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b][4 * r4 + e] = v4[e];
        }
      }
  }
  const float c2 = a.scale_log2;
  // V^T rows past d read zero
  if (D < DP)
    for (int i = tid; i < (BN / 4) * DP; i += NTHREADS)
      if (i % DP >= D) vt[i] = f32x4{};

  TileCursor<BN> cur = make_cursor<BN>(a, qg, wg_p_hi < wg_p0 ? -1 : wg_p_hi);
  if (wg_p_hi < wg_p0) cur.done = true;
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
  // per-lane LDS indices (float4 units) of the MFMA operands
  const int k_lane = (l32 >> 4) * 16 * NC + g * 16 + (l32 & 15);  // + 32 m: piece 2 m + g
  const int v_lane = g * DP + l32;                                  // + 2 DP j4 + 32 b: key quad 2 j4 + g

  for (; !cur.done && left > 0; --left) {
    __syncthreads();  // the previous tile's reads are done
    // stage K (blocked rows) and V (four keys to a float4); rows past the
    // segment end are zero
    for (int i = tid; i < BN * NC; i += NTHREADS) {
      const int r = i / NC, c = i - r * NC;
      const bool ok = cur.k0 + r < cur.kv_len;
      ks[(r >> 4) * 16 * NC + c * 16 + (r & 15)] =
          ok ? *(const f32x4*)(Kg + (cur.kv_row + cur.k0 + r) * a.k_ss + 4 * c) : f32x4{};
    }
    for (int i = tid; i < (BN / 4) * D; i += NTHREADS) {
      const int q4 = i / D, dv = i - q4 * D;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e;
        x[e] = cur.k0 + r < cur.kv_len ? Vg[(cur.kv_row + cur.k0 + r) * a.v_ss + dv] : 0.f;
      }
      vt[q4 * DP + dv] = x;
    }
    __syncthreads();

    // S^T: register r holds key k0 + 8 (r / 4) + 4 g + r % 4 of this lane's query
    f32x16 s = {};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const f32x4 kv = ks[k_lane + 32 * m];
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma(kv[e], qv[m][e], s);
    }
    int lim = cur.kv_len - 1 - cur.k0;
    if (a.causal) {
      const int lc = my_p + cur.delta - cur.k0;
      lim = lc < lim ? lc : lim;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * g + (r & 3);
      s[r] = kk > lim ? -INFINITY : s[r];
      mx = fmaxf(mx, s[r]);
    }
    mx = max_pair32(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < NDB; ++b) acc[b] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2f(fmaf(s[r], c2, -m_use));
      l_run += s[r];
    }
    // O^T += V^T P^T: product j' takes register j' of S^T
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const f32x4 vv = vt[v_lane + 2 * DP * j4 + 32 * b];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[b] = mfma(vv[e], s[4 * j4 + e], acc[b]);
      }
    cur.advance();
  }

  const float lt = sum_pair32(l_run);
  if (!row_ok) return;
  auto store_row = [&](float* row, float f) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv = 32 * b + 8 * r4 + 4 * g;
        if (dv < D) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[b][4 * r4 + e] * f;
          *(f32x4*)(row + dv) = v4;
        }
      }
  };
  if (a.mode == MODE_RING && a.kv_splits > 1) {
    // partial of this KV range: normalized o and natural lse
    const int64_t prow = (((int64_t)it.split * a.batch + it.b) * a.hq + h) * a.part_rows + qg.row_base + my_p;
    store_row(a.part_o + prow * D, lt > 0.f ? 1.f / lt : 0.f);
    if (g == 0) a.part_lse[prow] = lt > 0.f ? (m_run + log2f(lt)) * LN2 : -INFINITY;
  } else if (a.mode == MODE_RING) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = (int64_t)it.b * a.out_sb + (int64_t)h * a.out_sh + (qg.row_base + my_p) * a.out_ss;
    if (a.out_bf16) {
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dv = 32 * b + 8 * r4 + 4 * g;
          if (dv < D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ((__bf16*)a.out)[orow + dv + e] = (__bf16)(acc[b][4 * r4 + e] * inv);
          }
        }
    } else {
      store_row((float*)a.out + orow, inv);
    }
    if (a.lse != nullptr && g == 0) {
      const int64_t li = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
      a.lse[li] = lt > 0.f ? (m_run + log2f(lt)) * LN2 : -INFINITY;
    }
  } else {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
    if (g == 0) {
      a.m[mi] = m_run == m_in2 ? m_in : m_run * LN2;
      a.l[mi] = lt;
    }
    store_row(a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + my_p) * a.o_ss, 1.f);
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
  switch (a.d) {
    case 16: hipLaunchKernelGGL(attn_fwd_f32_kernel<16>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a); break;
    case 32: hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
