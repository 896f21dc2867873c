// Ring-ordered exact attention forward, bf16 inputs, d = 128, for gfx950.
//
// One workgroup = 4 waves (one per SIMD); each wave owns 64 query rows of one
// query head and keeps them on chip for the whole walk over the KV tiles:
//   * its Q tile as MFMA B operands in registers (64 rows x 128 = 64 VGPRs),
//   * the transposed output accumulator O^T (128 x 64 fp32 = 128 registers),
//   * the reference max m, the exact running max and the per-lane partial l.
// K and V tiles of 32 keys are staged once per workgroup through LDS (double
// buffered) and read by all 4 waves; with grouped-query attention the 4 waves
// are 4 query heads of one KV head, so every K/V byte fetched serves 4 heads.
//
// Per tile and wave (the online-softmax update of blockwise_attention /
// ring_attention_forward on the youngju.dev page and the m / l / o
// description of the "Context Parallelism" page):
//   S^T = K Q^T                 16 x v_mfma_f32_32x32x16_bf16
//   mask                        only tiles that cross the diagonal / segment end
//   m' = max(m, rowmax S)       in units of log2, c = scale * log2(e)
//   P  = 2^(S c - m')  l = 2^(m - m') l + rowsum P
//   O^T = 2^(m - m') O^T + V^T P^T   16 x v_mfma_f32_32x32x16_bf16
// The reference m is only moved when the tile maximum exceeds it by more than
// 2^8 (P stays below 256, harmless in fp32 and bf16), so the rescale of the
// 128 accumulator registers is skipped on almost every tile; the exact maximum
// is tracked on the side for the state handed back by the chunk entry point.
//
// Layout tricks:
//   * S is computed transposed (keys x queries): one query per lane, 16 keys
//     per lane, so the row max is in-lane plus one half-wave exchange and the
//     row sum needs no exchange until the end.
//   * The K rows fed to the QK MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that the 8 keys a lane holds per PV MFMA are 8 consecutive
//     keys; the V^T operand is then one 16-byte LDS read.
//   * V is transposed while it is staged (register 2x8 transposes with
//     v_perm_b32) so that V^T sits in LDS and both MFMA operands of every step
//     come from conflict-free ds_read_b128.
//   * K is copied global -> LDS directly (global_load_lds_dwordx4) with a
//     16-byte chunk swizzle chosen per lane.
#include <hip/hip_runtime.h>

#include "fwd_common.h"
#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int BN = 32;           // keys per tile
constexpr int WAVE_ROWS = 64;    // query rows per wave
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KROWB = D * 2;     // bytes of one K row in LDS
constexpr int VROWB = BN * 2;    // bytes of one V^T row (32 keys) in LDS
constexpr int KTILE = BN * KROWB;  // 8 KiB
constexpr int VTILE = D * VROWB;   // 8 KiB
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

// K tile: row-major, 16 chunks of 16 B per row; chunk c of row r is stored at
// c ^ kswz(r).  A K operand read touches 16 rows (mod 16 all distinct) at one
// chunk, so the swizzle spreads it over every bank.
__device__ __forceinline__ int kswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int k_off(int row, int chunk) { return row * KROWB + ((chunk ^ kswz(row)) << 4); }
// V^T tile: row dv holds 32 keys (4 chunks of 16 B); chunk c of row dv is
// stored at c ^ ((dv >> 2) & 3).  A V operand read touches 16 consecutive dv
// rows at one chunk: (dv mod 4, swizzled chunk) are then all distinct.
__device__ __forceinline__ int v_off(int dv, int chunk) { return dv * VROWB + ((chunk ^ ((dv >> 2) & 3)) << 4); }
// Row of the K tile that feeds MFMA row i of a 32-key block.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  // K0 K1 V0 V1
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * KTILE + 2 * VTILE];
  unsigned char* const kbuf0 = smem;
  unsigned char* const vbuf0 = smem + 2 * KTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;  // half-wave

  const WorkItem it = decode_work(a, blockIdx.x);
  const QGeom qg = query_geom(a, it);
  const int HP = a.heads_per_wg;
  const int G = a.hq / a.hkv;
  const int h = it.kvh * G + it.hg * HP + (wave % HP);
  const int wg_p0 = it.tile * a.rows_per_wg;
  const int p0 = wg_p0 + (wave / HP) * WAVE_ROWS;  // first row of this wave in the segment
  const int wg_p_hi = min(wg_p0 + a.rows_per_wg, qg.len) - 1;
  const int w_p_hi = min(p0 + WAVE_ROWS, qg.len) - 1;  // < p0 when the wave has no row

  const __bf16* Qg = (const __bf16*)a.q + (int64_t)it.b * a.q_sb + (int64_t)h * a.q_sh;
  const unsigned char* Kg = (const unsigned char*)a.k + ((int64_t)it.b * a.k_sb + (int64_t)it.kvh * a.k_sh) * 2;
  const unsigned char* Vg = (const unsigned char*)a.v + ((int64_t)it.b * a.v_sb + (int64_t)it.kvh * a.v_sh) * 2;
  const int64_t kss = a.k_ss * 2, vss = a.v_ss * 2;  // row strides in bytes

  // ---- Q tile as B operands: qf[qb][ks] = Q[row qb*32 + l32][ks*16 + 8g .. +8]
  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int p = p0 + qb * 32 + l32;
    const bool ok = p < qg.len;
    const __bf16* src = Qg + (qg.row_base + p) * a.q_ss + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[qb][ks] = ok ? *(const bf16x8*)(src + ks * 16) : bf16x8{};
  }

  // ---- running state (log2 units).  l_run is this half-wave's partial sum.
  float m_ref[2], m_max[2], l_run[2];
  f32x16 acc[4][2];  // acc[dvb][qb]: O^T[dv = dvb*32 + 8(r/4) + 4g + r%4][q = qb*32 + l32]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m_ref[qb] = -INFINITY;
    m_max[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb) acc[dvb][qb] = f32x16{};
  }
  if (a.mode == MODE_CHUNK) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int p = p0 + qb * 32 + l32;
      if (p < qg.len) {
        const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + p;
        const float mv = a.m[mi];
        m_ref[qb] = mv == -INFINITY ? -INFINITY : mv * LOG2E;
        m_max[qb] = m_ref[qb];
        l_run[qb] = g == 0 ? a.l[mi] : 0.f;
        const float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)p * a.o_ss;
#pragma unroll
        for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 v4 = *(const f32x4*)(orow + dvb * 32 + r4 * 8 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[dvb][qb][r4 * 4 + e] = v4[e];
          }
      }
    }
  }

  const float c2 = a.scale_log2;

  // ---- staging assignments
  // K: instruction i of wave w fills LDS rows 4(4i + w) .. +3; lane -> (row, stored chunk)
  const int k_row_in4 = lane >> 4;     // 0..3
  const int k_cpos = lane & 15;        // stored chunk position
  // V: thread -> dv chunk vc (dv 8vc .. 8vc+7) and key pair vk (keys 2vk, 2vk+1)
  const int vc = tid & 15;
  const int vk = tid >> 4;
  u32x4 vst[2];

  TileCursor<BN> cur = make_cursor<BN>(a, qg, wg_p_hi);
  if (wg_p_hi < wg_p0) cur.done = true;

  auto k_issue = [&](const TileCursor<BN>& c, unsigned char* kb) {
    const int last = c.kv_len - 1 - c.k0;  // last valid tile row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 4 * (4 * i + wave) + k_row_in4;
      const int src_row = row < last ? row : last;  // rows past the segment end repeat a valid row
      const int chunk = k_cpos ^ kswz(row);
      const unsigned char* src = Kg + (c.kv_row + c.k0 + src_row) * kss + chunk * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(kb + (4 * i + wave) * 1024), 16, 0, 0);
    }
  };
  auto v_load = [&](const TileCursor<BN>& c) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * vk + e;
      if (c.k0 + r < c.kv_len) vst[e] = *(const u32x4*)(Vg + (c.kv_row + c.k0 + r) * vss + vc * 16);
      else vst[e] = u32x4{0u, 0u, 0u, 0u};  // masked keys must meet finite V
    }
  };
  auto v_store = [&](unsigned char* vb) {
    // 2 keys x 8 dv -> 8 dv rows x 2 keys (4 bytes each)
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const unsigned ev = __builtin_amdgcn_perm(vst[1][pr], vst[0][pr], 0x05040100u);
      const unsigned od = __builtin_amdgcn_perm(vst[1][pr], vst[0][pr], 0x07060302u);
      const int dv_e = 8 * vc + 2 * pr;
      *(unsigned*)(vb + v_off(dv_e, vk >> 2) + 4 * (vk & 3)) = ev;
      *(unsigned*)(vb + v_off(dv_e + 1, vk >> 2) + 4 * (vk & 3)) = od;
    }
  };

  int buf = 0;
  if (!cur.done) {
    k_issue(cur, kbuf0);
    v_load(cur);
    v_store(vbuf0);
  }
  __syncthreads();

  TileCursor<BN> nxt = cur;
  if (!nxt.done) nxt.advance();

  while (!cur.done) {
    unsigned char* const kb = kbuf0 + buf * KTILE;
    unsigned char* const vb = vbuf0 + buf * VTILE;
    if (!nxt.done) {
      k_issue(nxt, kbuf0 + (buf ^ 1) * KTILE);
      v_load(nxt);
    }

    const int k0 = cur.k0;
    const bool wave_live = (w_p_hi >= p0) && !(a.causal && (int64_t)k0 - w_p_hi > cur.delta);
    if (wave_live) {
      // ---- S^T = K Q^T (K rows permuted by kperm)
      f32x16 s[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(kb + k_off(kperm(l32), 2 * ks + g));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[qb] = mfma(kf, qf[qb][ks], s[qb]);
      }

      // ---- mask.  Register r in half-wave g is tile key 16*(r/8) + 8g + r%8;
      //      it is hidden from row p when key > lim(p).
      const bool need_mask = (k0 + BN > cur.kv_len) ||
                             (a.causal && (int64_t)(k0 + BN - 1) - p0 > cur.delta);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int p = p0 + qb * 32 + l32;
          int64_t lim = (int64_t)cur.kv_len - 1 - k0;
          if (a.causal) {
            const int64_t lc = (int64_t)p + cur.delta - k0;
            lim = lc < lim ? lc : lim;
          }
          const int lim32 = (lim < -1 ? -1 : (int)lim) - 8 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 16 * (r >> 3) + (r & 7);
            s[qb][r] = kk > lim32 ? -INFINITY : s[qb][r];
          }
        }
      }

      // ---- online softmax
      float mx2[2];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
        mx = fmaxf(mx, xor32(mx));
        mx2[qb] = mx * c2;
        m_max[qb] = fmaxf(m_max[qb], mx2[qb]);
        grow |= mx2[qb] > m_ref[qb] + RESCALE_SLACK;  // also true when m_ref is -inf
      }
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = mx2[qb] > m_ref[qb] + RESCALE_SLACK ? mx2[qb] : m_ref[qb];
          const float alpha = m_ref[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
          m_ref[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int dvb = 0; dvb < 4; ++dvb) acc[dvb][qb] *= alpha;
        }
      }

      bf16x8 pf[2][2];  // pf[qb][m]: P^T B operand, tile keys 16m + 8g + 0..7
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_use = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
        float rs = 0.f;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[qb][mm * 8 + e], c2, -m_use));
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[qb][mm * 8 + e + 1], c2, -m_use));
            pf[qb][mm][e] = pr[0];
            pf[qb][mm][e + 1] = pr[1];
            rs = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, rs, false);
          }
        }
        l_run[qb] += rs;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dvb = 0; dvb < 4; ++dvb) {
          const bf16x8 vf = *(const bf16x8*)(vb + v_off(dvb * 32 + l32, 2 * mm + g));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) acc[dvb][qb] = mfma(vf, pf[qb][mm], acc[dvb][qb]);
        }
    }

    if (!nxt.done) v_store(vbuf0 + (buf ^ 1) * VTILE);
    __syncthreads();  // also waits for the direct-to-LDS K copies
    buf ^= 1;
    cur = nxt;
    if (!nxt.done) nxt.advance();
  }

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int p = p0 + qb * 32 + l32;
    float lt = l_run[qb] + xor32(l_run[qb]);
    if (p >= qg.len) continue;
    if (a.mode == MODE_RING) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t orow = (int64_t)it.b * a.out_sb + (int64_t)h * a.out_sh + (qg.row_base + p) * a.out_ss;
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dv = dvb * 32 + r4 * 8 + 4 * g;
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][qb][r4 * 4 + e] * inv;
          if (a.out_bf16) {
            bf16x4 b4;
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[e] = (__bf16)v4[e];
            *(bf16x4*)((__bf16*)a.out + orow + dv) = b4;
          } else {
            *(f32x4*)((float*)a.out + orow + dv) = v4;
          }
        }
      if (a.lse != nullptr && g == 0) {
        const int64_t li = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + p;
        a.lse[li] = lt > 0.f ? (m_ref[qb] + __log2f(lt)) * LN2 : -INFINITY;
      }
    } else {
      // hand back the state relative to the exact running maximum
      const float f = (m_max[qb] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[qb] - m_max[qb]);
      lt *= f;
      const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + p;
      if (g == 0) {
        a.m[mi] = m_max[qb] == -INFINITY ? -INFINITY : m_max[qb] * LN2;
        a.l[mi] = lt;
      }
      float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)p * a.o_ss;
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][qb][r4 * 4 + e] * f;
          *(f32x4*)(orow + dvb * 32 + r4 * 8 + 4 * g) = v4;
        }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(a.n_work), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ra
