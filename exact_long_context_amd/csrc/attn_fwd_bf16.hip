// Ring-ordered exact attention forward, bf16 inputs, d = 128, for gfx950.
//
// Workgroup = 8 waves, two per SIMD.  Each wave owns 32 query rows of one
// query head for the whole walk over the KV tiles and keeps on chip:
//   * its Q tile as MFMA B operands (32 rows x 128 bf16 = 32 VGPRs),
//   * the transposed output accumulator O^T (128 x 32 fp32 = 64 registers),
//   * the reference max m, the exact running max and a per-lane partial l.
// K and V tiles of 64 keys are staged once per workgroup through LDS and read
// by all 8 waves; with grouped-query attention the waves are the query heads
// of one KV head (4 heads x 64 rows), so each K/V byte fetched serves 4 heads.
//
// Per tile (the online-softmax update of blockwise_attention /
// ring_attention_forward on the youngju.dev page, and the m / l / o
// description of the "Context Parallelism" page), with c = scale * log2(e):
//   S^T = K Q^T                          16 x v_mfma_f32_32x32x16_bf16
//   mask (tiles crossing the diagonal or the segment end only)
//   m'  = max(m, c * rowmax S)           reference moved only when it grows by > 8
//   P   = 2^(c S - m'),  l = 2^(m - m') l + rowsum P
//   O^T = 2^(m - m') O^T + V^T P^T       16 x v_mfma_f32_32x32x16_bf16
// The reference m is moved only when the tile maximum exceeds it by more than
// 8 (so P < 256, harmless in fp32 and bf16); the O^T rescale therefore runs
// on few tiles.  The exact running maximum is tracked beside it for the state
// handed back by the chunk entry point.
//
// Software pipeline inside each wave, iteration j:
//   phase A: MFMA  S_{j+1} = K_{j+1} Q^T   ||  VALU  P_j = 2^(c S_j - m), rowsum
//   phase B: MFMA  O^T += V_j^T P_j^T      ||  VALU  mask / max of S_{j+1},
//                                                    V_{j+2} transpose into LDS
// so the exponentials of one tile hide under the matrix work of the next.
// LDS holds K for tiles j+1, j+2 and V^T for tiles j, j+1, j+2 (80 KiB).
//
// Layout tricks:
//   * S is computed transposed (keys x queries): one query per lane, 32 keys
//     per lane, so the row max is in-lane plus one half-wave exchange and the
//     row sum needs no exchange until the end.
//   * The K rows fed to the QK MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that the 8 keys a lane holds per PV MFMA are 8 consecutive
//     keys; the V^T operand is then one 16-byte LDS read.
//   * V is transposed while it is staged (2 keys x 8 dv register transposes
//     with v_perm_b32), so both MFMA operands come from ds_read_b128.
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

constexpr int D = 128;
constexpr int BN = 64;           // keys per tile
constexpr int WAVE_ROWS = 32;    // query rows per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KROWB = D * 2;       // bytes of one K row in LDS
constexpr int VROWB = BN * 2;      // bytes of one V^T row (64 keys) in LDS
constexpr int KTILE = BN * KROWB;  // 16 KiB
constexpr int VTILE = D * VROWB;   // 16 KiB
constexpr int NKBUF = 2, NVBUF = 3;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

// K tile: row-major, 16 chunks of 16 B per row; chunk c of row r is stored at
// c ^ kswz(r).  A K operand read touches 16 rows (all distinct mod 16) at one
// chunk, so the swizzle spreads it over every bank.
__device__ __forceinline__ int kswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int k_off(int row, int chunk) { return row * KROWB + ((chunk ^ kswz(row)) << 4); }
// V^T tile: row dv holds 64 keys (8 chunks of 16 B); chunk c of row dv is
// stored at c ^ ((dv >> 1) & 7).  A V operand read touches 16 consecutive dv
// rows at one chunk: (dv parity, swizzled chunk) are then all distinct.
__device__ __forceinline__ int v_off(int dv, int chunk) { return dv * VROWB + ((chunk ^ ((dv >> 1) & 7)) << 4); }
// Row of the K tile that feeds MFMA row i of a 32-key block.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

struct TileInfo {
  bool valid;
  int32_t k0, kv_len, delta;
  int64_t kv_row;
};

__device__ __forceinline__ TileInfo tile_info(const TileCursor<BN>& c) {
  TileInfo t;
  t.valid = !c.done;
  t.k0 = c.k0;
  t.kv_len = c.kv_len;
  t.delta = c.delta;
  t.kv_row = c.kv_row;
  return t;
}

__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NKBUF * KTILE + NVBUF * VTILE];
  unsigned char* const kbase = smem;
  unsigned char* const vbase = smem + NKBUF * KTILE;

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
  const int my_p = p0 + l32;                        // this lane's query row

  const __bf16* Qg = (const __bf16*)a.q + (int64_t)it.b * a.q_sb + (int64_t)h * a.q_sh;
  const unsigned char* Kg = (const unsigned char*)a.k + ((int64_t)it.b * a.k_sb + (int64_t)it.kvh * a.k_sh) * 2;
  const unsigned char* Vg = (const unsigned char*)a.v + ((int64_t)it.b * a.v_sb + (int64_t)it.kvh * a.v_sh) * 2;
  const int64_t kss = a.k_ss * 2, vss = a.v_ss * 2;  // row strides in bytes

  // ---- Q as B operands: qf[ks] = Q[row my_p][ks*16 + 8g .. +8]
  bf16x8 qf[8];
  {
    const bool ok = my_p < qg.len;
    const __bf16* src = Qg + (qg.row_base + my_p) * a.q_ss + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = ok ? *(const bf16x8*)(src + ks * 16) : bf16x8{};
  }

  // ---- running state (log2 units); l_run is this half-wave's partial sum
  float m_ref = -INFINITY, m_max = -INFINITY, l_run = 0.f;
  f32x16 acc[4];  // acc[dvb]: O^T[dv = dvb*32 + 8(r/4) + 4g + r%4][query my_p]
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb) acc[dvb] = f32x16{};
  if (a.mode == MODE_CHUNK && my_p < qg.len) {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + my_p;
    const float mv = a.m[mi];
    m_ref = mv == -INFINITY ? -INFINITY : mv * LOG2E;
    m_max = m_ref;
    l_run = g == 0 ? a.l[mi] : 0.f;
    const float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)my_p * a.o_ss;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v4 = *(const f32x4*)(orow + dvb * 32 + r4 * 8 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dvb][r4 * 4 + e] = v4[e];
      }
  }
  const float c2 = a.scale_log2;
  const bool causal = a.causal != 0;

  // ---- staging assignments
  // K: instruction i of wave w fills LDS rows 4(8i + w) .. +3; lane -> (row, stored chunk)
  const int k_row_in4 = lane >> 4;
  const int k_cpos = lane & 15;
  // V: thread -> dv chunk vc (dv 8vc .. 8vc+7) and key pair vk (keys 2vk, 2vk+1)
  const int vc = tid & 15;
  const int vk = tid >> 4;
  u32x4 vst[2];

  auto k_issue = [&](const TileInfo& t, unsigned char* kb) {
    const int last = t.kv_len - 1 - t.k0;  // last valid tile row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int grp = 8 * i + wave;
      const int row = 4 * grp + k_row_in4;
      const int src_row = row < last ? row : last;  // rows past the segment end repeat a valid row
      const int chunk = k_cpos ^ kswz(row);
      const unsigned char* src = Kg + (t.kv_row + t.k0 + src_row) * kss + chunk * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(kb + grp * 1024), 16, 0, 0);
    }
  };
  auto v_load = [&](const TileInfo& t) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * vk + e;
      if (t.k0 + r < t.kv_len) vst[e] = *(const u32x4*)(Vg + (t.kv_row + t.k0 + r) * vss + vc * 16);
      else vst[e] = u32x4{0u, 0u, 0u, 0u};  // masked keys must meet finite V
    }
  };
  auto v_store = [&](unsigned char* vb) {
    // 2 keys x 8 dv -> 8 dv rows x 2 keys (4 bytes each)
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const unsigned ev = __builtin_amdgcn_perm(vst[1][pr], vst[0][pr], 0x05040100u);
      const unsigned od = __builtin_amdgcn_perm(vst[1][pr], vst[0][pr], 0x07060302u);
      const int dv = 8 * vc + 2 * pr;
      *(unsigned*)(vb + v_off(dv, vk >> 2) + 4 * (vk & 3)) = ev;
      *(unsigned*)(vb + v_off(dv + 1, vk >> 2) + 4 * (vk & 3)) = od;
    }
  };

  // S^T of one tile for this wave: s[kb] covers keys kb*32 .. +31 (rows permuted by kperm)
  auto qk = [&](const unsigned char* kb, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        const bf16x8 kf = *(const bf16x8*)(kb + k_off(b2 * 32 + kperm(l32), 2 * ks + g));
        s[b2] = mfma(kf, qf[ks], s[b2]);
      }
  };
  // Mask a tile: register r of block b2 in half-wave g is tile key
  // b2*32 + 16*(r/8) + 8g + r%8; it is hidden from this lane's row when key > lim.
  auto apply_mask = [&](f32x16 (&s)[2], const TileInfo& t) {
    int64_t lim = (int64_t)t.kv_len - 1 - t.k0;
    if (causal) {
      const int64_t lc = (int64_t)my_p + t.delta - t.k0;
      lim = lc < lim ? lc : lim;
    }
    const int lim32 = (lim < -1 ? -1 : (lim > 1000 ? 1000 : (int)lim)) - 8 * g;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = b2 * 32 + 16 * (r >> 3) + (r & 7);
        s[b2][r] = kk > lim32 ? -INFINITY : s[b2][r];
      }
  };
  auto row_max = [&](const f32x16 (&s)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    mx = fmaxf(mx, xor32(mx));
    return mx * c2;
  };
  auto tile_needs_mask = [&](const TileInfo& t) -> bool {
    return (t.k0 + BN > t.kv_len) || (causal && (int64_t)(t.k0 + BN - 1) - p0 > t.delta);
  };
  // Move the reference maximum if the tile maximum mx2 outgrew it; rescales O^T and l.
  auto update_ref = [&](float mx2) {
    m_max = fmaxf(m_max, mx2);
    const bool grow = mx2 > m_ref + RESCALE_SLACK;  // also true when m_ref is -inf
    if (__any(grow)) {
      const float m_new = grow ? mx2 : m_ref;
      const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb) acc[dvb] *= alpha;
    }
  };
  // P^T B operands from S^T: pf[b2][mm] holds tile keys b2*32 + 16mm + 8g + 0..7
  auto softmax_p = [&](const f32x16 (&s)[2], bf16x8 (&pf)[2][2]) {
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float rs = 0.f;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pr;
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[b2][mm * 8 + e], c2, -m_use));
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[b2][mm * 8 + e + 1], c2, -m_use));
          pf[b2][mm][e] = pr[0];
          pf[b2][mm][e + 1] = pr[1];
          rs = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, rs, false);
        }
    l_run += rs;
  };
  auto pv = [&](const unsigned char* vb, const bf16x8 (&pf)[2][2]) {
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dvb = 0; dvb < 4; ++dvb) {
          const bf16x8 vf = *(const bf16x8*)(vb + v_off(dvb * 32 + l32, 4 * b2 + 2 * mm + g));
          acc[dvb] = mfma(vf, pf[b2][mm], acc[dvb]);
        }
  };

  // ---- tile stream: cur = j (softmax / PV), nx1 = j+1 (QK), nx2 = j+2 (loads)
  TileCursor<BN> nx2 = make_cursor<BN>(a, qg, wg_p_hi);
  if (wg_p_hi < wg_p0) nx2.done = true;
  TileInfo t_cur = tile_info(nx2);
  if (!nx2.done) nx2.advance();
  TileInfo t_nx1 = tile_info(nx2);
  if (!nx2.done) nx2.advance();

  if (t_cur.valid) {
    k_issue(t_cur, kbase);
    v_load(t_cur);
    v_store(vbase);
  }
  if (t_nx1.valid) {
    k_issue(t_nx1, kbase + KTILE);
    v_load(t_nx1);
    v_store(vbase + VTILE);
  }
  __syncthreads();

  f32x16 s_a[2], s_b[2];
  if (t_cur.valid) {
    qk(kbase, s_a);
    if (tile_needs_mask(t_cur)) apply_mask(s_a, t_cur);
    update_ref(row_max(s_a));
  }

  int kb_j = 0;  // K buffer of tile j (tile j+1 is in kb_j ^ 1)
  int vb_j = 0;  // V buffer of tile j (j+1 in (vb_j+1)%3, j+2 in (vb_j+2)%3)
  // one ring iteration; s_cur holds S^T of tile j (masked, reference updated)
  auto iteration = [&](f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    const TileInfo t_nx2 = tile_info(nx2);
    if (t_nx2.valid) {
      k_issue(t_nx2, kbase + kb_j * KTILE);  // K_j's buffer is free: QK(j) ran last iteration
      v_load(t_nx2);
    }
    // phase A: QK(j+1) || exponentials of tile j
    bf16x8 pf[2][2];
    qk(kbase + (kb_j ^ 1) * KTILE, s_nxt);
    softmax_p(s_cur, pf);
    if (t_nx1.valid && tile_needs_mask(t_nx1)) apply_mask(s_nxt, t_nx1);
    // phase B: PV(j) || max of tile j+1, V(j+2) transpose into LDS
    pv(vbase + vb_j * VTILE, pf);
    const float mx_next = row_max(s_nxt);
    v_store(vbase + (vb_j >= 1 ? vb_j - 1 : 2) * VTILE);  // (vb_j + 2) % 3; stale data if no tile j+2
    if (t_nx1.valid) update_ref(mx_next);
    __syncthreads();  // also waits for the direct-to-LDS K copies
    t_cur = t_nx1;
    t_nx1 = t_nx2;
    if (!nx2.done) nx2.advance();
    kb_j ^= 1;
    vb_j = vb_j == 2 ? 0 : vb_j + 1;
  };
  while (t_cur.valid) {
    iteration(s_a, s_b);
    if (!t_cur.valid) break;
    iteration(s_b, s_a);
  }

  // ---- epilogue
  float lt = l_run + xor32(l_run);
  if (my_p >= qg.len) return;
  if (a.mode == MODE_RING) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = (int64_t)it.b * a.out_sb + (int64_t)h * a.out_sh + (qg.row_base + my_p) * a.out_ss;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv = dvb * 32 + r4 * 8 + 4 * g;
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][r4 * 4 + e] * inv;
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
      const int64_t li = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
      a.lse[li] = lt > 0.f ? (m_ref + __log2f(lt)) * LN2 : -INFINITY;
    }
  } else {
    // hand back the state relative to the exact running maximum
    const float f = (m_max == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_max);
    lt *= f;
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + my_p;
    if (g == 0) {
      a.m[mi] = m_max == -INFINITY ? -INFINITY : m_max * LN2;
      a.l[mi] = lt;
    }
    float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)my_p * a.o_ss;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][r4 * 4 + e] * f;
        *(f32x4*)(orow + dvb * 32 + r4 * 8 + 4 * g) = v4;
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
