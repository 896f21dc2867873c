// Backward of ring-ordered exact attention, bf16 inputs, d = 128, for gfx950.
//
// The steps are those of ring_attention_backward on the youngju.dev page
// ("Ring Attention 논문 분석", backward listing): with D = rowsum(dO * O) and
// P = exp(s - lse) recomputed from the forward's log-sum-exp,
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D) scale,  dQ = dS K,  dK = dS^T Q.
// Three launches:
//   * bwd_prep: per query row, -lse / scale and -D into the workspace;
//   * attn_bwd_dq: per query tile (the forward's work decomposition), the KV
//     tiles in ring order; dQ stays on chip;
//   * attn_bwd_dkdv: per tile of 256 keys of one KV segment, every visible
//     query row of the requested query chunks, for every query head of the
//     KV head; dK and dV stay on chip, so their sums over the query heads and
//     the query chunks need no atomics.
// Every product is a v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and
// dS are rounded to bf16 as MFMA operands.
//
// Layouts in LDS: blocks of 16 rows, the 16-byte chunks of the 16 rows side
// by side (k_pos), so that an operand read takes 16 rows at one chunk; the
// per-step tiles also swap the rows inside a block by chunk (sw_pos: chunk c
// of row r at slot (r % 16) ^ 4 (c % 4)), so that one copy serves both the
// plain operand reads and the transposing ds_read_b64_tr_b16 reads (4 rows
// at 4 neighbouring chunk halves per 16 lanes) without bank conflicts.
// Tiles are filled by buffer loads that write LDS directly; rows past the end
// of their segment arrive as zeros.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "fwd_common.h"
#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int ROWB = 2 * D;          // bytes of one bf16 row
constexpr int TILE32 = 32 * ROWB;    // 8 KiB: 32 rows
constexpr int NTHREADS = 512;
constexpr float EMPTY_ROW = -1.0e30f;  // -lse / scale of a row that sees no key

__device__ __forceinline__ int k_pos(int row, int chunk) { return (row >> 4) * 4096 + chunk * 256 + (row & 15) * 16; }
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane byte offsets for the DMA of one 1 KiB block.
// k_pos tile: block blk (0..7 for 32 rows) = rows 16 (blk / 4) .. + 15, chunks 4 (blk % 4) .. + 3
__device__ __forceinline__ uint32_t nat_src(int blk, int lane, uint32_t rs) {
  return (uint32_t)(16 * (blk >> 2) + (lane & 15)) * rs + (uint32_t)(4 * (blk & 3) + (lane >> 4)) * 16;
}
// swizzled tile: the same blocks; the lane landing on slot lane % 16 of chunk c = 4 (blk % 4) + lane / 16
// fetches row (lane % 16) ^ 4 (c % 4) of the block, with c % 4 = lane / 16
__device__ __forceinline__ uint32_t sw_src(int blk, int lane, uint32_t rs) {
  return (uint32_t)(16 * (blk >> 2) + ((lane & 15) ^ ((lane >> 4) << 2))) * rs + (uint32_t)(4 * (blk & 3) + (lane >> 4)) * 16;
}

// One 16-byte-per-lane buffer load that writes LDS directly (lane l to byte 16 l of a 1 KiB block
// at dst), written out: the compiler does not track it, so it inserts no waits of its own before
// LDS reads it cannot tell apart from the load's target; the kernels wait for vmcnt themselves.
// dst is a wave-uniform LDS byte address.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_untracked(const void* base, uint32_t nrec, uint32_t dst, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nrec, 0x00020000);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Two transposing reads from a swizzled tile: lane 16 G + j gets rows 8 g .. 8 g + 3 (from lo) and
// 8 g + 4 .. 8 g + 7 (from hi) of column 32 dvb + 16 (G % 2) + j, i.e. an MFMA A operand (rows d,
// k = the tile's rows) with 8 consecutive rows along k; lo and hi come from tr_lane.
__device__ __forceinline__ bf16x8 tr_read(const unsigned char* lo_p, const unsigned char* hi_p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo_p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi_p);
  const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// Per-lane offset inside a swizzled tile of the transposing reads for d block 0 and rows 0..15
// (add 1024 dvb for d block dvb, 4096 for each further 16 rows): the lane supplies 4 columns
// 32 dvb + 16 (G % 2) + 4 (j % 4) .. + 3 of row 8 g + j / 4 (+ 4 for hi), from chunk
// 4 dvb + 2 (G % 2) + (j % 4) / 2, half j % 2.
__device__ __forceinline__ int tr_lane(int lane, int hi) {
  const int G = lane >> 4, j = lane & 15, g = lane >> 5;
  const int c3 = 2 * (G & 1) + ((j & 3) >> 1);
  return 256 * c3 + (((8 * g + (j >> 2) + 4 * hi) ^ (c3 << 2)) << 4) + 8 * (j & 1);
}
// Per-lane offset inside a swizzled tile of the plain operand read of tile row `row` (0..31; a
// further 32 rows add 8192) at chunk 2 ks + g, for a 16-d step ks of parity p (add 512 ks).
__device__ __forceinline__ int nat_lane(int row, int g, int p) {
  return (row >> 4) * 4096 + g * 256 + (((row & 15) ^ (8 * p + 4 * g)) << 4);
}

// ---------------------------------------------------------------------------
// prep: -lse / scale and -D per query row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const FwdArgs& f = a.f;
  const int64_t rows_total = (int64_t)f.batch * f.hq * a.q_rows;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;  // 8 of the 128 elements
  if (row >= rows_total) return;
  const int32_t r = (int32_t)(row % a.q_rows);
  const int64_t bh = row / a.q_rows;
  const int32_t h = (int32_t)(bh % f.hq), b = (int32_t)(bh / f.hq);
  const int64_t o = (int64_t)b * f.out_sb + (int64_t)h * f.out_sh + (int64_t)r * f.out_ss + 8 * sub;
  const bf16x8 dov = *(const bf16x8*)((const __bf16*)a.dout + o);
  float acc = 0.f;
  if (f.out_bf16) {
    const bf16x8 ov = *(const bf16x8*)((const __bf16*)f.out + o);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)dov[e], (float)ov[e], acc);
  } else {
    const f32x4 o0 = *(const f32x4*)((const float*)f.out + o);
    const f32x4 o1 = *(const f32x4*)((const float*)f.out + o + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf((float)dov[e], o0[e], fmaf((float)dov[e + 4], o1[e], acc)) ;
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (sub == 0) {
    const float lse = a.lse_in[(int64_t)b * f.ml_sb + (int64_t)h * f.ml_sh + r];
    a.w[row] = lse == -INFINITY ? EMPTY_ROW : -lse / a.scale;
    a.w[rows_total + row] = -acc;
  }
}

// ---------------------------------------------------------------------------
// dQ: per query tile, the KV tiles of 64 keys in ring order
// ---------------------------------------------------------------------------

constexpr int BNQ = 64;              // keys per tile
constexpr int NHALF = BNQ / 32;      // 32-key MFMA blocks per tile
constexpr int QTILE = BNQ * ROWB;    // bytes of one tile kind

__global__ __launch_bounds__(NTHREADS, 1) void attn_bwd_dq_kernel(BwdArgs a) {
  const FwdArgs& f = a.f;
  // Two buffers, each of K (read plainly for S^T = K Q^T and transposed for dQ^T += K^T dS^T) and V
  // (dP^T = V dO^T), swizzled tiles in one array: buffer B of tile kind T at (2 B + T) QTILE.  The
  // loop body is one tile with the buffer index a loop variable (two unrolled bodies made the
  // compiler copy the dQ accumulators between register sets on every tile); the loads are written
  // out (dma_untracked) and waited for explicitly, so the compiler adds no waits for them before the
  // operand reads.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * QTILE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const WorkItem it = decode_work(f, blockIdx.x);
  const QGeom qg = query_geom(f, it);
  const int HP = f.heads_per_wg;
  const int G = f.hq / f.hkv;
  const int h = it.kvh * G + it.hg * HP + (wave % HP);
  const int wg_p0 = it.tile * f.rows_per_wg;
  const int p0 = __builtin_amdgcn_readfirstlane(wg_p0 + (wave / HP) * 32);
  const int wg_p_hi = min(wg_p0 + f.rows_per_wg, qg.len) - 1;
  const int my_p = p0 + l32;
  const bool row_ok = my_p < qg.len;
  const int64_t qrow = qg.row_base + my_p;

  // Q and dO of this lane's query row as MFMA B operands
  bf16x8 qf[8], dof[8];
  {
    const __bf16* qs = (const __bf16*)f.q + (int64_t)it.b * f.q_sb + (int64_t)h * f.q_sh + qrow * f.q_ss + 8 * g;
    const __bf16* ds = (const __bf16*)a.dout + (int64_t)it.b * f.out_sb + (int64_t)h * f.out_sh + qrow * f.out_ss + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = row_ok ? *(const bf16x8*)(qs + 16 * ks) : bf16x8{};
      dof[ks] = row_ok ? *(const bf16x8*)(ds + 16 * ks) : bf16x8{};
    }
  }
  const float c2 = f.scale_log2;
  const int64_t wrow = ((int64_t)it.b * f.hq + h) * a.q_rows + qrow;
  const int64_t rows_total = (int64_t)f.batch * f.hq * a.q_rows;
  const float w1c = row_ok ? a.w[wrow] * c2 : 0.f;            // -lse log2(e)
  const float negD = row_ok ? a.w[rows_total + wrow] : 0.f;   // -D
  f32x16 negD16;  // the dP^T accumulator starts at -D (every register of a lane is its query row)
#pragma unroll
  for (int r = 0; r < 16; ++r) negD16[r] = negD;

  const unsigned char* Kg = (const unsigned char*)f.k + ((int64_t)it.b * f.k_sb + (int64_t)it.kvh * f.k_sh) * 2;
  const unsigned char* Vg = (const unsigned char*)f.v + ((int64_t)it.b * f.v_sb + (int64_t)it.kvh * f.v_sh) * 2;
  const uint32_t kss = (uint32_t)(f.k_ss * 2), vss = (uint32_t)(f.v_ss * 2);
  // DMA: wave w moves blocks w + 8 i (i < NHALF) of each of the two tiles
  uint32_t kn_src[NHALF], vn_src[NHALF];
#pragma unroll
  for (int i = 0; i < NHALF; ++i) {
    kn_src[i] = sw_src(wave + 8 * i, lane, kss);
    vn_src[i] = sw_src(wave + 8 * i, lane, vss);
  }
  const int blk_dst = __builtin_amdgcn_readfirstlane(wave * 1024);

  // plain operand reads (keys permuted), 16-d step ks: + 512 ks from the base of its parity
  const int k_lane0 = nat_lane(kperm(l32), g, 0), k_lane1 = nat_lane(kperm(l32), g, 1);
  const int t_lo = tr_lane(lane, 0), t_hi = tr_lane(lane, 1);  // transposing reads of K

  f32x16 acc[4];  // dQ^T[d = 32 dvb + 8 (r / 4) + 4 g + r % 4][query my_p]
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb) acc[dvb] = f32x16{};

  TileCursor<BNQ> cur = make_cursor<BNQ>(f, qg, wg_p_hi < wg_p0 ? -1 : wg_p_hi);
  if (wg_p_hi < wg_p0) cur.done = true;
  auto stage = [&](const TileCursor<BNQ>& c, int B) __attribute__((always_inline)) {
    const uint32_t nk = c.done ? 0u : (uint32_t)(c.kv_row + c.kv_len - 1) * kss + ROWB;
    const uint32_t nv = c.done ? 0u : (uint32_t)(c.kv_row + c.kv_len - 1) * vss + ROWB;
    const uint32_t sk = (uint32_t)(c.kv_row + c.k0) * kss, sv = (uint32_t)(c.kv_row + c.k0) * vss;
    const uint32_t base = lds0 + (uint32_t)(2 * B * QTILE + blk_dst);
#pragma unroll
    for (int i = 0; i < NHALF; ++i) {
      dma_untracked(Kg, nk, base + 8192 * i, kn_src[i], sk);
      dma_untracked(Vg, nv, base + QTILE + 8192 * i, vn_src[i], sv);
    }
  };

  auto compute = [&](const TileCursor<BNQ>& c, int B) __attribute__((always_inline)) {
    const unsigned char* kn = smem + 2 * B * QTILE;
    const unsigned char* vn = kn + QTILE;
    f32x16 s[NHALF], dp[NHALF];  // block hf: tile keys 32 hf ..; dp: dP^T - D
#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf) {
      s[hf] = f32x16{};
      dp[hf] = negD16;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf) {
        const int kl = (ks & 1) ? k_lane1 : k_lane0;
        s[hf] = mfma(*(const bf16x8*)(kn + kl + 8192 * hf + 512 * ks), qf[ks], s[hf]);
        dp[hf] = mfma(*(const bf16x8*)(vn + kl + 8192 * hf + 512 * ks), dof[ks], dp[hf]);
      }
    // register r of block hf holds tile key 32 hf + 16 (r / 8) + 8 g + r % 8; hide keys past the
    // segment end or the diagonal
    const bool need_mask = (c.k0 + BNQ > c.kv_len) || (c.causal && c.k0 + BNQ - 1 > c.delta + p0);
    if (need_mask) {
      int lim = c.kv_len - 1 - c.k0;
      if (c.causal) {
        const int lc = my_p + c.delta - c.k0;
        lim = lc < lim ? lc : lim;
      }
      lim = (lim < -1 ? -1 : (lim > 1000 ? 1000 : lim)) - 8 * g;
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * hf + 16 * (r >> 3) + (r & 7);
          s[hf][r] = kk > lim ? -INFINITY : s[hf][r];
        }
    }
    bf16x8 dsf[NHALF][2];  // dS^T as B operands: dsf[hf][st] holds keys 32 hf + 16 st + 8 g + 0..7
#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[hf][r], c2, w1c));
        dsf[hf][r >> 3][r & 7] = (__bf16)(p * dp[hf][r]);
      }
#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dvb = 0; dvb < 4; ++dvb) {
          const unsigned char* kt = kn + 1024 * dvb + 4096 * (st + 2 * hf);
          acc[dvb] = mfma(tr_read(kt + t_lo, kt + t_hi), dsf[hf][st], acc[dvb]);
        }
  };

  // double buffer: tile n in buffer n % 2; tile n + 1 is staged while tile n is computed
  if (!cur.done) stage(cur, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int B = 0; !cur.done; B ^= 1) {
    TileCursor<BNQ> nxt = cur;
    nxt.advance();
    if (!nxt.done) stage(nxt, B ^ 1);
    compute(cur, B);
    cur = nxt;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile n + 1 is in LDS
    __syncthreads();
  }

  if (!row_ok) return;
  float* dqrow = a.dq + (int64_t)it.b * f.q_sb + (int64_t)h * f.q_sh + qrow * f.q_ss;
  const float sc = a.scale;
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][r4 * 4 + e] * sc;
      *(f32x4*)(dqrow + dvb * 32 + r4 * 8 + 4 * g) = v4;
    }
}

// ---------------------------------------------------------------------------
// dK / dV: per 256 keys of one KV segment, the visible query rows in steps of 32
// ---------------------------------------------------------------------------

constexpr int KV_TILE = 256;  // keys per workgroup: 8 waves x 32
constexpr int BQ = 32;        // query rows per step

// Uniform walk over the steps of a workgroup: requested query chunk, its query
// segments, query row tiles of BQ, the query heads of the KV head.
struct StepCursor {
  int32_t ci, qs, hh, p0;   // query chunk index (relative), segment, head in group, first row
  int32_t qlen, p_start, p_top, delta, causal, kind_ok;
  int64_t q_row0;           // buffer row of the query segment's row 0
  bool done;
};

__global__ __launch_bounds__(NTHREADS, 1) void attn_bwd_dkdv_kernel(BwdArgs a) {
  const FwdArgs& f = a.f;
  // One LDS array with explicit offsets.  The per-step tiles (two buffers each of Q, read plainly
  // for S = Q K^T and transposed for dK^T += Q^T dS, and of dO, read plainly for dP = dO V^T and
  // transposed for dV^T += dO^T P; swizzled tiles) sit in the first 32 KiB, where every operand
  // address is one register plus an instruction offset; V of the workgroup's 256 keys (k_pos
  // layout, for the whole launch) and the per-row terms follow.  The step loads are written out
  // (dma_untracked) and waited for explicitly.
  constexpr int QN = 0, ON = 2 * TILE32;         // + B * TILE32
  constexpr int VS = 4 * TILE32;                 // 32 KiB
  constexpr int WT = VS + KV_TILE * ROWB;        // + B * 256: -lse / scale, then -D, of the step's rows
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WT + 512];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t nseg = num_segments(f.layout);
  const int32_t L = f.lq;
  // work item: (b, kvh, KV chunk j, segment sb, key tile kt).  When the KV
  // streams (batch x KV head) split evenly over the 8 XCDs, workgroup w lands
  // on XCD w % 8 with the other workgroups of its stream: they all walk the
  // same query and dO rows (the query heads of one KV head), so that XCD's L2
  // serves their tiles and no other XCD fetches them.
  const int32_t per_stream = f.n_chunks * nseg * a.kv_tiles_per_seg;
  const int32_t n_streams = f.batch * f.hkv;
  int32_t w, stream;
  if (n_streams % 8 == 0) {
    const int32_t u = (int32_t)blockIdx.x >> 3;
    stream = ((int32_t)blockIdx.x & 7) + 8 * (u / per_stream);
    w = u % per_stream;
  } else {
    stream = (int32_t)blockIdx.x / per_stream;
    w = (int32_t)blockIdx.x % per_stream;
  }
  const int32_t kt = w % a.kv_tiles_per_seg; w /= a.kv_tiles_per_seg;
  const int32_t sb = w % nseg; w /= nseg;
  const int32_t j = w;
  const int32_t kvh = stream % f.hkv;
  const int32_t b = stream / f.hkv;
  const Segment kseg = segment_l(f.layout, L, f.n_chunks, j, sb);
  const int64_t k_row0 = (int64_t)j * L + kseg.row0;  // buffer row of the segment's row 0
  const int32_t kv_len = kseg.len;
  const int32_t k_lo = kt * KV_TILE;                    // first key of the workgroup (segment rows)
  const int32_t kw0 = k_lo + 32 * wave;                 // first key of this wave
  const int32_t my_k = kw0 + l32;
  const bool key_ok = my_k < kv_len;
  const bool wave_live = kw0 < kv_len;
  const int G = f.hq / f.hkv;

  const uint32_t vss = (uint32_t)(f.v_ss * 2);
  const uint32_t qss = (uint32_t)(f.q_ss * 2), oss = (uint32_t)(f.out_ss * 2);
  const unsigned char* Kg = (const unsigned char*)f.k + ((int64_t)b * f.k_sb + (int64_t)kvh * f.k_sh) * 2;
  const unsigned char* Vg = (const unsigned char*)f.v + ((int64_t)b * f.v_sb + (int64_t)kvh * f.v_sh) * 2;

  // K of this lane's key as MFMA B operands (S = Q K^T: B = K^T, lane = key)
  bf16x8 kf[8];
  {
    const __bf16* ks = (const __bf16*)(Kg) + (k_row0 + my_k) * f.k_ss + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = key_ok ? *(const bf16x8*)(ks + 16 * s) : bf16x8{};
  }
  // V of the workgroup's keys into LDS (8 blocks per wave; rows past the segment end read zero)
  {
    const uint32_t nv = (uint32_t)(k_row0 + kv_len - 1) * vss + ROWB;
    const uint32_t sv = (uint32_t)(k_row0 + k_lo) * vss;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int blk = 8 * wave + i;  // rows 16 (blk / 4) .., chunks 4 (blk % 4) ..
      dma_untracked(Vg, nv, lds0 + VS + blk * 1024, nat_src(blk, lane, vss), sv);
    }
  }

  const float c2 = f.scale_log2;
  const int64_t rows_total = (int64_t)f.batch * f.hq * a.q_rows;
  const uint32_t w_bytes = (uint32_t)(2 * rows_total * 4);
  // plain operand reads (query rows permuted), 16-d step ks: + 512 ks from the base of its parity
  const int q_lane0 = nat_lane(kperm(l32), g, 0), q_lane1 = nat_lane(kperm(l32), g, 1);
  // V as B operand (lane = key): + 512 s; the per-row terms of the step (lanes read 8 g ..)
  const unsigned char* vb_addr = smem + VS + k_pos(32 * wave + l32, g);
  const unsigned char* w_lane = smem + WT;
  const int t_lo = tr_lane(lane, 0), t_hi = tr_lane(lane, 1);  // transposing reads of Q and dO
  const uint32_t qn_src = sw_src(wave, lane, qss), on_src = sw_src(wave, lane, oss);
  const int blk_dst = __builtin_amdgcn_readfirstlane(wave * 1024);

  f32x16 acck[4], accv[4];  // dK^T / dV^T[d = 32 dvb + 8 (r / 4) + 4 g + r % 4][key my_k]
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb) acck[dvb] = accv[dvb] = f32x16{};

  // ---- step walk
  auto load_seg = [&](StepCursor& c) __attribute__((always_inline)) {
    // set up query segment (ci, qs); kind_ok = 0 when no row of it sees a key of the workgroup
    const int32_t qchunk = f.q_first + c.ci;
    const Segment qseg = segment_l(f.layout, L, f.n_chunks, qchunk, c.qs);
    c.qlen = qseg.len;
    c.q_row0 = (int64_t)c.ci * L + qseg.row0;
    int64_t dl = f.causal ? pair_delta(qseg, kseg) : 0;
    const int64_t lim = (int64_t)1 << 30;
    c.delta = (int32_t)(dl > lim ? lim : (dl < -lim ? -lim : dl));
    int64_t ps = 0;
    if (f.causal) {
      ps = (int64_t)k_lo - dl;  // key k_lo is visible from query row k_lo - delta on
      ps = ps < 0 ? 0 : ps;
    }
    c.kind_ok = (k_lo < kv_len) && (ps < c.qlen);
    // row tiles aligned to BQ, walked from the segment end down: the
    // workgroups of one KV head then stream the same query rows at about the
    // same time whatever their first visible row (rows below it are masked)
    c.p_start = (int32_t)(ps < c.qlen ? ps : c.qlen) / BQ * BQ;
    c.p_top = (c.qlen - 1) / BQ * BQ;
    c.p0 = c.p_top;
    c.hh = 0;
  };
  auto skip_empty = [&](StepCursor& c) __attribute__((always_inline)) {
    while (!c.done && !c.kind_ok) {
      if (++c.qs >= nseg) { c.qs = 0; ++c.ci; }
      if (c.ci >= f.q_count) { c.done = true; break; }
      load_seg(c);
    }
  };
  // inside a query segment: row tiles from the top down, the heads of the
  // group inner, so that all workgroups walk the same rows in step
  auto advance = [&](StepCursor& c) __attribute__((always_inline)) {
    if (++c.hh < G) return;
    c.hh = 0;
    c.p0 -= BQ;
    if (c.p0 < c.p_start) {
      c.kind_ok = 0;  // next segment
      skip_empty(c);
    }
  };
  StepCursor cur;
  cur.ci = 0; cur.qs = 0; cur.done = false; cur.causal = f.causal;
  load_seg(cur);
  skip_empty(cur);

  auto stage = [&](const StepCursor& c, auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    const int h = kvh * G + c.hh;
    const unsigned char* Qg = (const unsigned char*)f.q + ((int64_t)b * f.q_sb + (int64_t)h * f.q_sh) * 2;
    const unsigned char* Og = (const unsigned char*)a.dout + ((int64_t)b * f.out_sb + (int64_t)h * f.out_sh) * 2;
    const int64_t end = c.q_row0 + c.qlen - 1;
    const uint32_t nq = (uint32_t)end * qss + ROWB, no = (uint32_t)end * oss + ROWB;
    const uint32_t sq = (uint32_t)(c.q_row0 + c.p0) * qss, so = (uint32_t)(c.q_row0 + c.p0) * oss;
    dma_untracked(Qg, nq, lds0 + QN + B * TILE32 + blk_dst, qn_src, sq);
    dma_untracked(Og, no, lds0 + ON + B * TILE32 + blk_dst, on_src, so);
    if (wave == 0 && lane < 16) {
      // lanes 0..7: -lse / scale of the 32 rows; lanes 8..15: -D
      const uint32_t row = (uint32_t)(((int64_t)b * f.hq + h) * a.q_rows + c.q_row0 + c.p0);
      const uint32_t off = (row + 4 * (lane & 7)) * 4 + (lane >= 8 ? (uint32_t)(rows_total * 4) : 0u);
      dma_untracked(a.w, w_bytes, lds0 + WT + B * 256, off, 0u);
    }
  };

  auto compute = [&](const StepCursor& c, auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    const unsigned char* qn = smem + QN + B * TILE32;
    const unsigned char* on = smem + ON + B * TILE32;
    const float* wt = (const float*)(w_lane + B * 256);
    // register r of lane (key l32, g) holds query row 16 (r / 8) + 8 g + r % 8 of the step
    f32x16 s, dp;
    {
      const f32x4 a0 = *(const f32x4*)(wt + 8 * g), a1 = *(const f32x4*)(wt + 8 * g + 4);
      const f32x4 a2 = *(const f32x4*)(wt + 16 + 8 * g), a3 = *(const f32x4*)(wt + 16 + 8 * g + 4);
      const f32x4 b0 = *(const f32x4*)(wt + BQ + 8 * g), b1 = *(const f32x4*)(wt + BQ + 8 * g + 4);
      const f32x4 b2 = *(const f32x4*)(wt + BQ + 16 + 8 * g), b3 = *(const f32x4*)(wt + BQ + 16 + 8 * g + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = a0[e]; s[4 + e] = a1[e]; s[8 + e] = a2[e]; s[12 + e] = a3[e];
        dp[e] = b0[e]; dp[4 + e] = b1[e]; dp[8 + e] = b2[e]; dp[12 + e] = b3[e];
      }
    }
    // S + (-lse / scale) and dP + (-D)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int ql = (ks & 1) ? q_lane1 : q_lane0;
      s = mfma(*(const bf16x8*)(qn + ql + 512 * ks), kf[ks], s);
      dp = mfma(*(const bf16x8*)(on + ql + 512 * ks), *(const bf16x8*)(vb_addr + 512 * ks), dp);
    }
    // hide rows past the segment end and pairs past the diagonal
    const bool need_mask = (c.p0 + BQ > c.qlen) || (c.causal && kw0 + 31 - c.p0 > c.delta);
    if (need_mask) {
      const int hi = c.qlen - c.p0 - 8 * g;                       // rows >= hi are past the end
      const int lo = c.causal ? my_k - c.p0 - c.delta - 8 * g : -1000000;  // rows < lo are before the key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qo = 16 * (r >> 3) + (r & 7);
        s[r] = (qo >= hi || qo < lo) ? -INFINITY : s[r];
      }
    }
    bf16x8 pb[2], db[2];  // P and dS as B operands: [st] holds query rows 16 st + 8 g + 0..7
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] * c2);
      pb[r >> 3][r & 7] = (__bf16)p;
      db[r >> 3][r & 7] = (__bf16)(p * dp[r]);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb) {
        const int o = 1024 * dvb + 4096 * st;
        accv[dvb] = mfma(tr_read(on + o + t_lo, on + o + t_hi), pb[st], accv[dvb]);
        acck[dvb] = mfma(tr_read(qn + o + t_lo, qn + o + t_hi), db[st], acck[dvb]);
      }
  };

  if (!cur.done) stage(cur, std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0x0F70);  // V and the first step are in LDS
  __syncthreads();
  auto step = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    StepCursor nxt = cur;
    advance(nxt);
    if (!nxt.done) stage(nxt, std::integral_constant<int, B ^ 1>{});
    if (wave_live) compute(cur, bc);
    cur = nxt;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  while (!cur.done) {
    step(std::integral_constant<int, 0>{});
    if (cur.done) break;
    step(std::integral_constant<int, 1>{});
  }

  if (!key_ok) return;
  const int64_t krow = k_row0 + my_k;
  float* dkrow = a.dk + (int64_t)b * f.k_sb + (int64_t)kvh * f.k_sh + krow * f.k_ss;
  float* dvrow = a.dv + (int64_t)b * f.v_sb + (int64_t)kvh * f.v_sh + krow * f.v_ss;
  const float sc = a.scale;
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 k4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = acck[dvb][r4 * 4 + e] * sc;
        v4[e] = accv[dvb][r4 * 4 + e];
      }
      *(f32x4*)(dkrow + dvb * 32 + r4 * 8 + 4 * g) = k4;
      *(f32x4*)(dvrow + dvb * 32 + r4 * 8 + 4 * g) = v4;
    }
}

// Workspace of the entry point that allocates nothing (ra_ring_bwd_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the GPU concerned.
static __device__ __align__(256) unsigned char scratch[BWD_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t bwd_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows_total = (int64_t)a.f.batch * a.f.hq * a.q_rows;
  if (rows_total <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows_total + 15) / 16)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.f.n_work <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(a.f.n_work), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.n_work_kv <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(a.n_work_kv), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ra
