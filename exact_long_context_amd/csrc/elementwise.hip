// Memory-bound kernels of the library: state initialization, finalize, the
// log-sum-exp merge of two partials, and the layout permutation.
//
// Row kernels give each row to a group of d/8 consecutive lanes, each lane
// moving 8 fp32 values (two 16-byte pieces) of the row, so a wave touches
// 2 KiB of consecutive fp32 state (coalesced) and reads every per-row scalar
// once per lane group, before any lane of that group writes (which makes the
// in-place merge safe).  Eight values per lane measured 10 % faster than four
// for finalize and state init; finalize also streams o with non-temporal
// loads (8 % faster; non-temporal stores slowed merge and state init).
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int ROW_THREADS = 256;

struct RowIdx {
  bool ok;
  int64_t ml;   // index into m / l / lse
  int64_t o;    // index of this lane's 4 floats in o
  int64_t out;  // index of this lane's 4 elements in out
  int c4;       // which 8-element piece
};

__device__ __forceinline__ RowIdx row_index(const RowsArgs& g) {
  const int lpr = g.d >> 3;  // lanes per row
  const int64_t t = (int64_t)blockIdx.x * ROW_THREADS + threadIdx.x;
  const int64_t row = t / lpr;
  RowIdx r;
  r.c4 = (int)(t - row * lpr);
  const int64_t total = (int64_t)g.batch * g.heads * g.rows;
  r.ok = row < total;
  const int64_t bh = row / g.rows;
  const int64_t p = row - bh * g.rows;
  const int64_t b = bh / g.heads, h = bh - b * g.heads;
  r.ml = b * g.ml_sb + h * g.ml_sh + p;
  r.o = b * g.o_sb + h * g.o_sh + p * g.o_ss + 8 * r.c4;
  r.out = b * g.out_sb + h * g.out_sh + p * g.out_ss + 8 * r.c4;
  return r;
}

__global__ __launch_bounds__(ROW_THREADS) void state_init_kernel(RowsArgs g, float* m, float* l, float* o) {
  const RowIdx r = row_index(g);
  if (!r.ok) return;
  if (r.c4 == 0) {
    m[r.ml] = -INFINITY;
    l[r.ml] = 0.f;
  }
  *(f32x4*)(o + r.o) = f32x4{0.f, 0.f, 0.f, 0.f};
  *(f32x4*)(o + r.o + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(ROW_THREADS) void finalize_kernel(RowsArgs g, const float* m, const float* l,
                                                               const float* o, void* out, int out_bf16,
                                                               float* lse) {
  const RowIdx r = row_index(g);
  if (!r.ok) return;
  const float lv = l[r.ml];
  const bool seen = lv > 0.f;
  const float inv = seen ? 1.f / lv : 0.f;
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)(o + r.o)) * inv;
  const f32x4 w = __builtin_nontemporal_load((const f32x4*)(o + r.o + 4)) * inv;
  if (out_bf16) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) { b[e] = (__bf16)v[e]; b[4 + e] = (__bf16)w[e]; }
    *(bf16x8*)((__bf16*)out + r.out) = b;
  } else {
    *(f32x4*)((float*)out + r.out) = v;
    *(f32x4*)((float*)out + r.out + 4) = w;
  }
  if (lse != nullptr && r.c4 == 0) lse[r.ml] = seen ? m[r.ml] + logf(lv) : -INFINITY;
}

__global__ __launch_bounds__(ROW_THREADS) void merge_kernel(RowsArgs g, const float* lse_a, const float* o_a,
                                                            const float* lse_b, const float* o_b, float* lse_out,
                                                            float* o_out) {
  const RowIdx r = row_index(g);
  if (!r.ok) return;
  const float la = lse_a[r.ml], lb = lse_b[r.ml];
  const f32x4 va = *(const f32x4*)(o_a + r.o), va2 = *(const f32x4*)(o_a + r.o + 4);
  const f32x4 vb = *(const f32x4*)(o_b + r.o), vb2 = *(const f32x4*)(o_b + r.o + 4);
  const float M = fmaxf(la, lb);
  float lse, wa, wb;
  if (M == -INFINITY) {
    lse = -INFINITY; wa = 0.f; wb = 0.f;
  } else {
    const float ea = expf(la - M), eb = expf(lb - M);  // exp(-inf) = 0
    const float tot = ea + eb;
    lse = M + logf(tot);
    wa = ea / tot;
    wb = eb / tot;
  }
  *(f32x4*)(o_out + r.o) = va * wa + vb * wb;
  *(f32x4*)(o_out + r.o + 4) = va2 * wa + vb2 * wb;
  if (r.c4 == 0) lse_out[r.ml] = lse;
}

// Split-KV partials -> out, lse (the log-sum-exp associativity of the
// lecture 013 notes, over all S partials at once).  Partial s of row
// (b, h, p) sits at row ((s B + b) H + h) rows + p of part_lse / part_o
// (contiguous).  Every lane of a row group reads the row's S log-sum-exps;
// the weights are taken against their maximum, so the sum is exact up to
// rounding in any order of s.
__global__ __launch_bounds__(ROW_THREADS) void split_merge_kernel(RowsArgs g, int32_t S, const float* part_lse,
                                                                  const float* part_o, void* out, int out_bf16,
                                                                  float* lse) {
  const RowIdx r = row_index(g);
  if (!r.ok) return;
  const int lpr = g.d >> 3;
  const int64_t row = ((int64_t)blockIdx.x * ROW_THREADS + threadIdx.x) / lpr;  // (b H + h) rows + p
  const int64_t plane = (int64_t)g.batch * g.heads * g.rows;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_lse[s * plane + row]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, acc2 = acc;
  float tot = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float w = expf(part_lse[s * plane + row] - M);  // exp(-inf) = 0
      tot += w;
      const float* src = part_o + (s * plane + row) * g.d + 8 * r.c4;
      acc += *(const f32x4*)src * w;
      acc2 += *(const f32x4*)(src + 4) * w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const f32x4 v = acc * inv, v2 = acc2 * inv;
  if (out_bf16) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) { b[e] = (__bf16)v[e]; b[4 + e] = (__bf16)v2[e]; }
    *(bf16x8*)((__bf16*)out + r.out) = b;
  } else {
    *(f32x4*)((float*)out + r.out) = v;
    *(f32x4*)((float*)out + r.out + 4) = v2;
  }
  if (lse != nullptr && r.c4 == 0) lse[r.ml] = tot > 0.f ? M + logf(tot) : -INFINITY;
}

// Permutation: physical row c*L + p  <->  logical row pos(c, p).  Each thread
// moves one UNIT-byte piece; a workgroup covers consecutive pieces of one
// (batch, head) so that reads and writes of a row stay together.
template <typename UNIT>
__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a, const UNIT* __restrict__ src,
                                                      UNIT* __restrict__ dst) {
  const int64_t per_bh = a.seq * a.units_per_row;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= per_bh) return;
  const int64_t phys = t / a.units_per_row;
  const int64_t u = t - phys * a.units_per_row;
  const int64_t L = a.seq / a.n_chunks;
  const int32_t c = (int32_t)(phys / L);
  const int64_t logical = position(a.layout, a.seq, a.n_chunks, c, phys - (int64_t)c * L);
  const int64_t src_row = a.to_chunked ? logical : phys;
  const int64_t dst_row = a.to_chunked ? phys : logical;
  // (batch, head) pairs: grid rows, strided when there are more than the grid has
  for (int64_t bh = blockIdx.y; bh < a.batch * a.heads; bh += gridDim.y) {
    const int64_t b = bh / a.heads, h = bh - b * a.heads;
    dst[b * a.dst_sb + h * a.dst_sh + dst_row * a.dst_ss + u] =
        src[b * a.src_sb + h * a.src_sh + src_row * a.src_ss + u];
  }
}

inline unsigned blocks_for(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

}  // namespace

hipError_t launch_state_init(const RowsArgs& g, float* m, float* l, float* o, hipStream_t stream) {
  const int64_t threads = (int64_t)g.batch * g.heads * g.rows * (g.d >> 3);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(state_init_kernel, dim3(blocks_for(threads, ROW_THREADS)), dim3(ROW_THREADS), 0, stream, g, m,
                     l, o);
  return hipGetLastError();
}

hipError_t launch_finalize(const RowsArgs& g, const float* m, const float* l, const float* o, void* out,
                           int32_t out_bf16, float* lse, hipStream_t stream) {
  const int64_t threads = (int64_t)g.batch * g.heads * g.rows * (g.d >> 3);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(blocks_for(threads, ROW_THREADS)), dim3(ROW_THREADS), 0, stream, g, m,
                     l, o, out, out_bf16, lse);
  return hipGetLastError();
}

hipError_t launch_merge(const RowsArgs& g, const float* lse_a, const float* o_a, const float* lse_b,
                        const float* o_b, float* lse_out, float* o_out, hipStream_t stream) {
  const int64_t threads = (int64_t)g.batch * g.heads * g.rows * (g.d >> 3);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks_for(threads, ROW_THREADS)), dim3(ROW_THREADS), 0, stream, g, lse_a,
                     o_a, lse_b, o_b, lse_out, o_out);
  return hipGetLastError();
}

hipError_t launch_split_merge(const RowsArgs& g, int32_t kv_splits, const float* part_lse, const float* part_o,
                              void* out, int32_t out_bf16, float* lse, hipStream_t stream) {
  const int64_t threads = (int64_t)g.batch * g.heads * g.rows * (g.d >> 3);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(split_merge_kernel, dim3(blocks_for(threads, ROW_THREADS)), dim3(ROW_THREADS), 0, stream, g,
                     kv_splits, part_lse, part_o, out, out_bf16, lse);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& p, int unit, const void* src, void* dst, hipStream_t stream) {
  const int64_t per_bh = p.seq * p.units_per_row;
  const int64_t bh = p.batch * p.heads;
  if (per_bh == 0 || bh == 0) return hipSuccess;
  const dim3 grid(blocks_for(per_bh, 256), (unsigned)(bh < 65535 ? bh : 65535)), block(256);
  switch (unit) {
    case 16:
      hipLaunchKernelGGL(permute_kernel<uint4>, grid, block, 0, stream, p, (const uint4*)src, (uint4*)dst);
      break;
    case 8:
      hipLaunchKernelGGL(permute_kernel<uint2>, grid, block, 0, stream, p, (const uint2*)src, (uint2*)dst);
      break;
    case 4:
      hipLaunchKernelGGL(permute_kernel<uint32_t>, grid, block, 0, stream, p, (const uint32_t*)src, (uint32_t*)dst);
      break;
    case 2:
      hipLaunchKernelGGL(permute_kernel<uint16_t>, grid, block, 0, stream, p, (const uint16_t*)src, (uint16_t*)dst);
      break;
    default:
      hipLaunchKernelGGL(permute_kernel<uint8_t>, grid, block, 0, stream, p, (const uint8_t*)src, (uint8_t*)dst);
      break;
  }
  return hipGetLastError();
}

}  // namespace ra
